// Append path: hot-window append with FIFO eviction, and the quantiser that
// writes evicted tokens into cold code tiles.
//
// Codec: "TurboQuant: kompresja KV-cache w LLM 6 razy" (sudonull.com),
// section "Zasada dzialania PolarQuant" (random rotation, then radius and
// angle per pair, then quantisation) and section "Kompensacja bledow przez
// QJL" (1-bit Johnson-Lindenstrauss sketch of the residual).
// Eviction: "Monarch v3: Paginacion KV Inspirada en NES", section "Como
// funciona" (sliding window: the newest tokens stay hot, older ones go cold)
// and the decode loop's evict-oldest-to-cold step.
//
// Three kernels per append launch, in stream order:
//   k_append_plan  one thread per sequence: FIFO bookkeeping; lists evicted
//                  NEW ring entries, revives tombstones of evicted PROMOTED
//                  entries, assigns cold slots and ring positions.
//   k_quantize     one wave per (cold tile, sequence, kv head, K or V) item,
//                  persistent blocks with Pi and S staged in LDS: rotation on
//                  MFMA (16x16x32 f16, Pi split into fp16 hi + lo/2^12, fp32
//                  accumulate), pair codes in registers, residual sketch on
//                  MFMA (S and the unit residual both split hi/lo), packing
//                  through LDS into the K and V tile layouts.
//   k_hot_append   copies the input tokens that stay hot into the ring.
#include "tq_device.h"
#include "tq_promote_body.h"
#include "tq_qprep_body.h"

namespace tq {

__global__ void k_clear(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_clear(void* p, size_t bytes, hipStream_t st) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
    k_clear<<<blocks, 256, 0, st>>>(reinterpret_cast<uint32_t*>(p), n);
    return hipGetLastError();
}

// FIFO step of one sequence's append, read from the state only: evicts the
// oldest hot entries beyond the window (NEW ones are listed in jobs for
// quantisation, PROMOTED ones in revive: their tombstoned cold slot comes
// back), assigns cold slots and ring positions.
struct PlanView {
    AppendPlan pl;
    int e;           // hot entries and input tokens evicted
    int head2;       // ring index of the oldest hot entry afterwards
    int count2;      // hot entries afterwards
    int n_revive;    // PROMOTED entries evicted
    int overflow;    // the cold region is full (host capacity checks make this unreachable)
};

// m: the (sequence, layer) metadata; tags: its ring tags (global or LDS).
__device__ PlanView plan_view(const Dims& dm, const SeqLayerMeta& m, const int* tags, const CallSeqs& cs, int bi,
                              int* jobs, int* revive, int rstep) {
    const int n = cs.n_new[bi];
    const int h = m.count, head = m.head, nc = m.cold_len;
    const int e = max(0, h + n - dm.W);
    const int e_ring = min(e, h);
    int e_in = e - e_ring;
    int k = 0, nr = 0;
    for (int i = 0; i < e_ring; ++i) {
        const int phys = (head + i) % dm.cap;
        const int tag = tags[phys];
        if (tag < 0)
            jobs[k++] = phys;
        else
            revive[rstep * nr++] = tag;
    }
    PlanView v;
    v.pl.nc_old = nc;
    v.pl.in_base = cs.in_base[bi];
    // (the tensor-cache tier writes evicted tokens into its matrix, no slots)
    v.overflow = !dm.tc && nc + k + e_in > dm.cold_cap;
    if (v.overflow) {
        k = 0;
        e_in = 0;
    }
    v.pl.n_ring_new = k;
    v.pl.e_in = e_in;
    v.head2 = (head + e_ring) % dm.cap;
    const int live = h - e_ring;
    v.pl.ring_pos = (v.head2 + live) % dm.cap;
    v.pl.n_keep = n - (e - e_ring);
    v.pl.nc_new = dm.tc ? nc : nc + k + e_in;
    v.pl.pad = 0;
    v.e = e;
    v.count2 = live + v.pl.n_keep;
    v.n_revive = nr;
    return v;
}

// Writes a planned FIFO step into the state (metadata, revived cold slots).
__device__ void plan_commit(const Dims& dm, const Ptrs& P, int layer, int seq, const PlanView& v, const int* revive,
                            int rstep) {
    const size_t sl = sl_index(dm, seq, layer);
    SeqLayerMeta* m = P.meta + sl;
    uint32_t* tomb = P.tomb + sl * (dm.cold_cap / 32);
    uint32_t* stk = P.sticky + sl * dm.cold_cap;
    for (int i = 0; i < v.n_revive; ++i) {
        const int tag = revive[rstep * i];
        tomb[tag >> 5] &= ~(1u << (tag & 31));
        stk[tag] = 0u;
    }
    if (v.overflow) atomicOr(P.err, DEVERR_COLD_OVERFLOW);
    m->head = v.head2;
    m->count = v.count2;
    m->cold_len = v.pl.nc_new;
    m->n_evicted += v.e;
}

__global__ void k_append_plan(Dims dm, Ptrs P, int layer, CallSeqs cs) {
    if (threadIdx.x != 0) return;
    const int bi = blockIdx.x;
    // the revived slots share the jobs buffer: NEW entries from the front,
    // PROMOTED ones from the back (at most cap entries are evicted in all)
    int* jobs = P.jobs + (size_t)bi * dm.cap;
    const size_t sl = sl_index(dm, cs.ids[bi], layer);
    const PlanView v = plan_view(dm, P.meta[sl], P.tags + sl * dm.cap, cs, bi, jobs, jobs + dm.cap - 1, -1);
    plan_commit(dm, P, layer, cs.ids[bi], v, jobs + dm.cap - 1, -1);
    P.plan[bi] = v.pl;
}

// Kept input tokens into the ring: one block per (32 kept tokens, sequence,
// kv head).  K rows are copied 16 bytes per thread.  A group that fills one
// whole ring tile also goes through LDS for its V tile, whose rows (one per
// component) hold the 32 tokens in storage order: each thread writes 16-byte
// row pieces.  Other groups (a ring position not on a tile edge, or the last
// partial group) write V one value at a time.
template <int D>
__global__ __launch_bounds__(256) void k_hot_append(Dims dm, Ptrs P, int layer, CallSeqs cs,
                                                    const _Float16* __restrict__ in_k,
                                                    const _Float16* __restrict__ in_v) {
    constexpr int CPT = D / 8;  // 16-byte pieces per token row
    __shared__ __attribute__((aligned(16))) _Float16 s_v[TILE][D + 8];
    const int bi = blockIdx.y, kvh = blockIdx.z, tid = threadIdx.x;
    const AppendPlan pl = P.plan[bi];
    const int t0 = blockIdx.x * TILE;
    if (t0 >= pl.n_keep) return;
    const int nt = min(TILE, pl.n_keep - t0);
    const int seq = cs.ids[bi];
    const int tok0 = pl.in_base + (cs.n_new[bi] - pl.n_keep) + t0;
    const int phys0 = (pl.ring_pos + t0) % dm.cap;
    const size_t rb = ring_base(dm, seq, layer, kvh);
    const bool tile_run = nt == TILE && phys0 % TILE == 0;
    for (int i = tid; i < nt * CPT; i += 256) {
        const int t = i / CPT, c = i % CPT;
        const size_t src = ((size_t)(tok0 + t) * dm.hkv + kvh) * D + 8 * c;
        const int phys = (phys0 + t) % dm.cap;
        *reinterpret_cast<uint4*>(P.ring_k + rb + (size_t)phys * D + 8 * c) =
            *reinterpret_cast<const uint4*>(in_k + src);
        const uint4 v = *reinterpret_cast<const uint4*>(in_v + src);
        if (tile_run) {
            *reinterpret_cast<uint4*>(&s_v[t][8 * c]) = v;
        } else {
            const _Float16* vh = reinterpret_cast<const _Float16*>(&v);
            _Float16* dst = P.ring_v + rb + (size_t)(phys / TILE) * D * TILE + vpos(phys % TILE);
#pragma unroll
            for (int r = 0; r < 8; ++r) dst[(size_t)(8 * c + r) * TILE] = vh[r];
        }
    }
    if (tile_run) {
        __syncthreads();
        // row k of the V tile, storage positions 8 j .. 8 j + 7
        _Float16* vt = P.ring_v + rb + (size_t)(phys0 / TILE) * D * TILE;
        for (int i = tid; i < D * (TILE / 8); i += 256) {
            const int k = i / (TILE / 8), j = i % (TILE / 8);
            half8 w;
#pragma unroll
            for (int r = 0; r < 8; ++r) w[r] = s_v[vtok(8 * j + r)][k];
            *reinterpret_cast<half8*>(vt + (size_t)k * TILE + 8 * j) = w;
        }
    }
    if (kvh == 0 && tid < nt) P.tags[sl_index(dm, seq, layer) * dm.cap + (phys0 + tid) % dm.cap] = -1;
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// v_writelane_b32: lane `lane` of the result takes the wave-uniform `value`,
// the other lanes keep `old` (the compiler's intrinsic, reached by name)
__device__ int writelane_i32(int value, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// 32 codes of CB bits, one per byte of the 32 bytes (a, b) (first code in
// the low byte of a.x), packed at bit i CB of w, least significant first.
template <int CB>
__device__ __forceinline__ void pack32(const uint4& a, const uint4& b, uint32_t (&w)[CB]) {
    const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < CB; ++k) w[k] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t c = (u[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const int bit = i * CB, k = bit >> 5, sh = bit & 31;
        w[k] |= c << sh;
        if (sh + CB > 32) w[k + 1] |= c >> (32 - sh);
    }
}

// Quantiser launch: persistent blocks of QNT threads.  An item is the 32 K or
// the 32 V vectors of one (cold tile, sequence, kv head); each wave takes
// items in a stride over the launch and packs them itself.  Pi and S (fp16 hi
// and lo parts) are staged in LDS once per block, so the MFMA A operands of
// every item come from LDS.  Lane l of a wave owns vectors l % 16 and
// 16 + l % 16 of its item and, of every 16-component tile of a rotated
// vector, components 4 (l / 16) .. +3 (the MFMA accumulator layout).
constexpr int QNT = 512;

template <int D, int CB, int M>
__global__ __launch_bounds__(QNT) void k_quantize(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs,
                                                  const _Float16* __restrict__ in_k,
                                                  const _Float16* __restrict__ in_v) {
    constexpr int PAIRS = D / 2;
    constexpr int NCT = D / 16;
    constexpr int NKB = D / 32;
    constexpr int NJT = M / 16;
    constexpr int NB = D / 8;  // 16-byte blocks per fp16 row
    constexpr int NW = QNT / 64;
    static_assert((D * NB) % 64 == 0 && (M * NB) % 64 == 0, "whole waves of 16-byte copies");
    __shared__ __attribute__((aligned(16))) _Float16 s_ph[D * D];  // Pi hi rows (blocks swizzled)
    __shared__ __attribute__((aligned(16))) _Float16 s_pl[D * D];  // Pi lo rows
    __shared__ __attribute__((aligned(16))) _Float16 s_sh[M * D];  // S hi rows (MFMA column order)
    __shared__ __attribute__((aligned(16))) _Float16 s_sl[M * D];  // S lo rows
    __shared__ __attribute__((aligned(16))) uint8_t s_code[NW][TILE][PAIRS];  // a wave's codes (layout: see below)
    __shared__ uint2 s_mask[NW][2 * (M / 16) * 4];                           // a wave's sign masks
    __shared__ float2 s_unit[1 << CB];          // code c = a | b << rb: a (cos, sin) of grid angle b turned by half a bin
    __shared__ int s_pref[MAX_CALL_SEQ + 1];  // items before each sequence
    __shared__ int4 s_plan[MAX_CALL_SEQ];     // nc_old, nc_new, n_ring_new, in_base

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: item bookkeeping stays scalar
    const int q = lane >> 4, n16 = lane & 15;
    constexpr int TB = theta_bits_of(CB), RB = CB - TB, LR = 1 << RB;
    // The turned copies of Pi and S for TB angle bits: the rotation yields
    // every pair turned by half an angle bin, the angle code is then read off
    // signs alone, the residual is formed in the turned frame (its norm is
    // the same) and S T^T sketches it as S does the unturned one.
    const _Float16* pi_hi = P.tpi_hi + (size_t)(TB - 2) * D * D;
    const _Float16* pi_lo = P.tpi_lo + (size_t)(TB - 2) * D * D;
    const _Float16* sk_hi = P.ts_hi + (size_t)(TB - 2) * M_MAX * D;
    const _Float16* sk_lo = P.ts_lo + (size_t)(TB - 2) * M_MAX * D;
    // Pi and S into LDS, 16 bytes per lane: row r's block c sits at slot
    // c ^ (r % NB), so the 16 rows of an operand tile, read at one block,
    // hit different banks.
    {
        auto copy = [&](const _Float16* g, _Float16* lds, int nblk) {
            for (int p0 = 64 * wave; p0 < nblk; p0 += QNT) {
                const int pos = p0 + lane, r = pos / NB, c = pos % NB;
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(g) + r * NB + (c ^ (r & (NB - 1))),
                                                 (__attribute__((address_space(3))) void*)(lds + 8 * p0), 16, 0, 0);
            }
        };
        copy(pi_hi, s_ph, D * NB);
        copy(pi_lo, s_pl, D * NB);
        copy(sk_hi, s_sh, M * NB);
        copy(sk_lo, s_sl, M * NB);
    }
    for (int c = tid; c < (1 << CB); c += QNT) {
        const float a = (float)(c & ((1 << F.rb) - 1));
        const int b = c >> F.rb;
        s_unit[c] = make_float2(a * F.cos_h[b], a * F.sin_h[b]);
    }
    // items of each sequence: the tiles its new cold slots touch, times kv
    // heads, times K and V
    if (wave == 0) {
        int carry = 0;
        for (int b0 = 0; b0 < cs.n; b0 += 64) {
            const int b = b0 + lane;
            int c = 0;
            if (b < cs.n) {
                const AppendPlan pl = P.plan[b];
                if (pl.nc_new > pl.nc_old) c = ((pl.nc_new + TILE - 1) / TILE - pl.nc_old / TILE) * dm.hkv * 2;
                s_plan[b] = make_int4(pl.nc_old, pl.nc_new, pl.n_ring_new, pl.in_base);
            }
            int x = c;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            if (b < cs.n) s_pref[b + 1] = carry + x;
            carry += __shfl(x, 63, 64);
        }
        if (lane == 0) s_pref[0] = 0;
    }
    __syncthreads();

    const int n_items = s_pref[cs.n];
    int bi = 0;
    for (int it = blockIdx.x * NW + wave; it < n_items; it += gridDim.x * NW) {
        while (it >= s_pref[bi + 1]) ++bi;
        const int4 pl = s_plan[bi];  // nc_old, nc_new, n_ring_new, in_base
        const int rr = it - s_pref[bi];
        const int kv = rr & 1, kvh = (rr >> 1) % dm.hkv, tile = pl.x / TILE + (rr >> 1) / dm.hkv;
        const int seq = cs.ids[bi];
        const int lo = max(pl.x, tile * TILE), hi = min(pl.y, tile * TILE + TILE);

        // source vectors: evicted ring entries or input rows
        half8 xb[2][NKB];
        bool valid[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int slot = tile * TILE + 16 * g + n16;
            valid[g] = slot >= lo && slot < hi;
            const _Float16* src = nullptr;
            int stride = 1;
            if (valid[g]) {
                const int rel = slot - pl.x;
                if (rel < pl.z) {
                    const int phys = P.jobs[(size_t)bi * dm.cap + rel];
                    const size_t rb = ring_base(dm, seq, layer, kvh);
                    if (kv == 0) {
                        src = P.ring_k + rb + (size_t)phys * D;
                    } else {
                        src = P.ring_v + rb + (size_t)(phys / 32) * D * 32 + vpos(phys % 32);
                        stride = 32;
                    }
                } else {
                    const size_t row = ((size_t)(pl.w + rel - pl.z) * dm.hkv + kvh) * D;
                    src = (kv == 0 ? in_k : in_v) + row;
                }
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if (!valid[g]) {
#pragma unroll
                    for (int r = 0; r < 8; ++r) xb[g][kb][r] = (_Float16)0.0f;
                } else if (stride == 1) {
                    xb[g][kb] = *reinterpret_cast<const half8*>(src + kb * 32 + 8 * q);
                } else {
#pragma unroll
                    for (int r = 0; r < 8; ++r) xb[g][kb][r] = src[(size_t)(kb * 32 + 8 * q + r) * 32];
                }
            }
        }

        // rotation y = T Pi x (pairs turned), one 16-row tile at a time for both vector groups
        float y[2][NCT][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int row = ct * 16 + n16;
            half8 ah[NKB], al[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int off = row * D + 8 * ((4 * kb + q) ^ (row & (NB - 1)));
                ah[kb] = *reinterpret_cast<const half8*>(s_ph + off);
                al[kb] = *reinterpret_cast<const half8*>(s_pl + off);
            }
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                floatx4 acc_h = {0.f, 0.f, 0.f, 0.f}, acc_l = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    acc_h = mfma16x16x32(ah[kb], xb[g][kb], acc_h);
                    acc_l = mfma16x16x32(al[kb], xb[g][kb], acc_l);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) y[g][ct][r] = acc_h[r] + acc_l[r] * (1.0f / LO_SCALE);
            }
        }

        // per vector: R = fp16(max pair radius) over its four lanes, pair
        // codes, residual e and rho = fp16(|e|).  The sketch takes the
        // residual times (L_r - 1) / R (the signs do not depend on its scale),
        // split into fp16 hi and lo parts.  Codes go to LDS in the order the
        // packing reads them: K by token in record order, V by pair in
        // storage order.
        uint8_t* cb = &s_code[wave][0][0];
        _Float16 R16[2], rho16[2];
        half8 eh[2][NKB], el[2][NKB];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int t = 16 * g + n16;
            float rad[NCT][2];
            float rmax = 0.0f;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float a = y[g][ct][2 * h], b = y[g][ct][2 * h + 1];
                    rad[ct][h] = __builtin_amdgcn_sqrtf(a * a + b * b);
                    rmax = fmaxf(rmax, rad[ct][h]);
                }
            }
            rmax = fmaxf(rmax, __shfl_xor(rmax, 16, 64));
            rmax = fmaxf(rmax, __shfl_xor(rmax, 32, 64));
            R16[g] = (_Float16)rmax;
            float R = (float)R16[g];
            if (!(R <= 65504.0f)) {
                if (valid[g] && q == 0) atomicOr(P.err, DEVERR_R_OVERFLOW);
                R = 65504.0f;
            }
            // hardware reciprocal (within 1 ulp): the level decision moves by
            // less than the boundary band's width
            const float inv = R > 0.0f ? (float)(LR - 1) * __builtin_amdgcn_rcpf(R) : 0.0f;  // 0 for R = 0: every code a = 0
            const float stepr = R * (1.0f / (float)(LR - 1));
            float e[NCT][4];
            float esq = 0.0f;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                uint32_t c2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float a0 = y[g][ct][2 * h], a1 = y[g][ct][2 * h + 1];
                    // nearest level (a tie at exactly half a step is inside the band)
                    const int a = (int)fminf(rad[ct][h] * inv + 0.5f, (float)(LR - 1));
                    const int b = angle_sector_t<TB>(a0, a1);
                    c2[h] = (uint32_t)(a | (b << RB));
                    const float2 u = s_unit[c2[h]];
                    const float e0 = a0 - stepr * u.x, e1 = a1 - stepr * u.y;
                    e[ct][2 * h] = e0;
                    e[ct][2 * h + 1] = e1;
                    esq += e0 * e0 + e1 * e1;
                }
                if (kv == 0) {
                    // pairs 8 ct + 2 q + h sit at record positions p0 + h
                    const int p0 = (D / 8) * (2 * (ct & 1) + (q >> 1)) + 4 * (ct >> 1) + 2 * (q & 1);
                    *reinterpret_cast<uint16_t*>(cb + t * PAIRS + p0) = (uint16_t)(c2[0] | (c2[1] << 8));
                } else {
                    cb[(8 * ct + 2 * q) * TILE + vpos(t)] = (uint8_t)c2[0];
                    cb[(8 * ct + 2 * q + 1) * TILE + vpos(t)] = (uint8_t)c2[1];
                }
            }
            esq += __shfl_xor(esq, 16, 64);
            esq += __shfl_xor(esq, 32, 64);
            rho16[g] = (_Float16)__builtin_amdgcn_sqrtf(esq);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 8; r += 2) {
                    float v0 = e[2 * kb + (r >> 2)][r & 3] * inv, v1 = e[2 * kb + (r >> 2)][(r & 3) + 1] * inv;
                    pin(v0);
                    pin(v1);
                    const float2v v = {v0, v1};
                    const half2v hv = __builtin_convertvector(v, half2v);
                    // lo = fp16((v - hi) 2^12) as one mixed-precision fma per
                    // component: hi 2^12 is exact in fp16 (|v| < 16), and
                    // v 2^12 - hi 2^12 is exact in fp32, so the only rounding
                    // is the final one to fp16
                    const half2v hs = hv * (half2v){(_Float16)LO_SCALE, (_Float16)LO_SCALE};
                    eh[g][kb][r] = hv[0];
                    eh[g][kb][r + 1] = hv[1];
                    el[g][kb][r] = (_Float16)fmaf(v0, LO_SCALE, -(float)hs[0]);
                    el[g][kb][r + 1] = (_Float16)fmaf(v1, LO_SCALE, -(float)hs[1]);
                }
            }
        }

        // sketch signs: z = S_m e, one 16-row tile of S at a time.  Sign
        // (jt, r) of the 16 vectors of group g, over the four lane quarters,
        // is one wave-wide mask: bit 16 q + n is sign 16 jt + 4 q + r of
        // vector 16 g + n.
        constexpr int NMASK = 2 * NJT * 4;
        const uint64_t vmask[2] = {__builtin_amdgcn_ballot_w64(valid[0]), __builtin_amdgcn_ballot_w64(valid[1])};
        uint32_t mlo = 0, mhi = 0;  // lane i < NMASK: mask i = (g NJT + jt) 4 + r
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
            const int row = jt * 16 + n16;
            half8 sh[NKB], sl[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int off = row * D + 8 * ((4 * kb + q) ^ (row & (NB - 1)));
                sh[kb] = *reinterpret_cast<const half8*>(s_sh + off);
                sl[kb] = *reinterpret_cast<const half8*>(s_sl + off);
            }
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                floatx4 z1 = {0.f, 0.f, 0.f, 0.f}, z2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    z1 = mfma16x16x32(sh[kb], eh[g][kb], z1);
                    z2 = mfma16x16x32(sh[kb], el[g][kb], z2);
                    z2 = mfma16x16x32(sl[kb], eh[g][kb], z2);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float z = z1[r] + z2[r] * (1.0f / LO_SCALE);
                    const uint64_t m = __builtin_amdgcn_ballot_w64(z >= 0.0f) & vmask[g];
                    const int i = (g * NJT + jt) * 4 + r;
                    mlo = (uint32_t)writelane_i32((int)(uint32_t)m, i, (int)mlo);
                    mhi = (uint32_t)writelane_i32((int)(uint32_t)(m >> 32), i, (int)mhi);
                }
            }
        }
        if (lane < NMASK) s_mask[wave][lane] = make_uint2(mlo, mhi);

        uint8_t* base = P.cold + cold_tile_offset(dm, F, seq, kvh, kv, tile);
        uint8_t* meta = base + TILE * (F.pb + F.sb);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int vec = 16 * g + n16;
            if (valid[g] && q == 0) {
                *reinterpret_cast<_Float16*>(meta + 2 * vec) = R16[g];
                *reinterpret_cast<_Float16*>(meta + 2 * TILE + 2 * (kv == 0 ? vec : vpos(vec))) = rho16[g];
            }
        }
        // the codes and masks written above are read back by other lanes of
        // this wave (its LDS operations complete in order)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // pack: a lane packs 32 codes (a K record's half or a V pair row)
        // into CB words with fixed shifts, and one sign word from the masks.
        // A tile only partly covered by this launch keeps its other tokens'
        // bits: V words are OR-ed in.
        const bool full = lo == tile * TILE && hi == tile * TILE + TILE;
        constexpr int PB = PAIRS * CB / 8;
        if (kv == 0) {
            constexpr int LPT = PAIRS / 32;  // lanes per token
            if (lane < TILE * LPT) {
                const int t = lane / LPT, part = lane % LPT;
                const uint4* src = reinterpret_cast<const uint4*>(cb + t * PAIRS + 32 * part);
                uint32_t w[CB];
                pack32<CB>(src[0], src[1], w);
                const int st = tile * TILE + t;
                if (st >= lo && st < hi) {
                    uint32_t* dst = reinterpret_cast<uint32_t*>(base + t * PB + part * 4 * CB);
#pragma unroll
                    for (int k = 0; k < CB; ++k) dst[k] = w[k];
                }
            }
            // K sign word w of token t = 16 g + n: bits 16 jt' + 4 q + r from
            // bit 16 q + n of mask (g, 2 w + jt', r)
            constexpr int SW = M / 32;
            if (lane < TILE * SW) {
                const int t = lane / SW, sw = lane % SW, g = t >> 4, n = t & 15;
                const uint2* mk = &s_mask[wave][(g * NJT + 2 * sw) * 4];
                uint32_t word = 0;
#pragma unroll
                for (int jh = 0; jh < 2; ++jh) {
                    uint32_t x = 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint2 m = mk[jh * 4 + r];
                        // quarters 0, 1 from the low word (bits n, 16 + n), 2, 3 from the high word
                        const uint32_t b = ((m.x >> n) & 0x10001u) | (((m.y >> n) & 0x10001u) << 8);
                        x |= b << r;  // quarter q's four bits at 0, 16, 8, 24 for q = 0, 1, 2, 3
                    }
                    const uint32_t h16 = (x & 0x0F0Fu) | ((x >> 12) & 0xF0F0u);  // quarter q at bits 4 q
                    word |= h16 << (16 * jh);
                }
                const int st = tile * TILE + t;
                if (st >= lo && st < hi) reinterpret_cast<uint32_t*>(base + TILE * PB + t * (M / 8))[sw] = word;
            }
        } else {
            if (lane < PAIRS) {
                const uint4* src = reinterpret_cast<const uint4*>(cb + lane * TILE);
                uint4 u0 = src[0], u1 = src[1];
                if (!full) {
                    // codes are computed for every slot of the tile: keep those of this launch's tokens
                    const uint32_t tm = (hi - tile * TILE >= 32 ? 0xffffffffu : (1u << (hi - tile * TILE)) - 1u) &
                                        ~((1u << (lo - tile * TILE)) - 1u);
                    uint32_t bm[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        bm[i] = 0;
#pragma unroll
                        for (int k = 0; k < 4; ++k) bm[i] |= ((tm >> vtok(4 * i + k)) & 1u) ? (0xffu << (8 * k)) : 0u;
                    }
                    u0 = make_uint4(u0.x & bm[0], u0.y & bm[1], u0.z & bm[2], u0.w & bm[3]);
                    u1 = make_uint4(u1.x & bm[4], u1.y & bm[5], u1.z & bm[6], u1.w & bm[7]);
                }
                uint32_t w[CB];
                pack32<CB>(u0, u1, w);
                uint32_t* dst = reinterpret_cast<uint32_t*>(base + (size_t)lane * 4 * CB);
#pragma unroll
                for (int k = 0; k < CB; ++k) {
                    if (full)
                        dst[k] = w[k];
                    else if (w[k])
                        atomicOr(dst + k, w[k]);
                }
            }
            // V sign plane j: bit s = vpos(16 g + n) = 8 (n / 4) + 4 g + n % 4
            // from bit 16 q + n of mask (g, j / 16, j % 4), q = (j / 4) % 4
            if (lane < M) {
                const int jt = lane >> 4, qq = (lane >> 2) & 3, r = lane & 3;
                uint32_t plane = 0;
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const uint2 m = s_mask[wave][(g * NJT + jt) * 4 + r];
                    uint32_t x = ((qq & 2) ? m.y : m.x) >> (16 * (qq & 1)) & 0xFFFFu;
                    x = (x | (x << 8)) & 0x00FF00FFu;
                    x = (x | (x << 4)) & 0x0F0F0F0Fu;  // nibble k of the 16 bits -> byte k
                    plane |= x << (4 * g);
                }
                uint32_t* dst = reinterpret_cast<uint32_t*>(base + TILE * PB) + lane;
                if (full)
                    *dst = plane;
                else if (plane)
                    atomicOr(dst, plane);
            }
        }
        // the next item's LDS writes stay after this item's reads
        __builtin_amdgcn_wave_barrier();
    }
}

// Small appends (a few tokens per sequence, as in a decode step): one block
// per (sequence, kv head).  Every block of a sequence derives the FIFO step
// from the same state, reading only; each quantises the K and V vectors of
// its kv head's evicted NEW entries and writes the kept tokens into its
// ring; the last block of the sequence to finish commits the step (metadata,
// ring tags, revived cold slots).  Thread (vector slot s, component i) of a
// pass over NT / D vectors:
//   rotation  y_i = <row i of Pi, x> in fp32, four partial sums over the
//             input index mod 4 (row i, read as column i of Pi^T, is held in
//             registers; S is copied to LDS by global-to-LDS loads; both are
//             requested together with the planning's loads)
//   codes     the pair (2p, 2p + 1) sits on adjacent lanes; R = fp16(max
//             radius over the vector's pairs), pair codes, residual e and
//             rho = fp16(|e|)
//   sketch    thread (s, j < m): sign j = [<S_j, e> >= 0] (S in LDS)
//   packing   the wave of threads (s, 0 .. 63): the slot's K record or V rows
template <int D, int CB, int M>
__device__ __forceinline__ void append_small_body(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                                                  const CallSeqs& cs, const _Float16* __restrict__ in_k,
                                                  const _Float16* __restrict__ in_v) {
    constexpr int NT = 256;
    constexpr int PAIRS = D / 2;
    constexpr int PB = PAIRS * CB / 8;
    constexpr int SB = M / 8;
    constexpr int VP = NT / D;   // vectors per pass
    constexpr int WPV = D / 64;  // waves per vector
    constexpr int XS = D + 4;    // padded LDS rows (16-byte reads of different rows hit different banks)
    static_assert(M <= 64 && M <= D, "one sketch row per thread of the vector's first wave");
    __shared__ PlanView s_pv;
    constexpr int NB = D / 4;    // 16-byte blocks per row
    __shared__ __attribute__((aligned(16))) float s_s[M][D];   // S rows (blocks swizzled)
    __shared__ __attribute__((aligned(16))) float s_x[VP][XS]; // input vectors
    __shared__ __attribute__((aligned(16))) float s_e[VP][XS]; // residuals
    __shared__ uint32_t s_code[VP][PAIRS];
    __shared__ float s_red[2][NT / 64];
    __shared__ float s_cos[16], s_sin[16];
    __shared__ __attribute__((aligned(16))) SeqLayerMeta s_meta;
    __shared__ int s_last;
    extern __shared__ int s_dyn[];  // [cap] ring tags, [cap] jobs, [cap] revived slots
    int* s_tags = s_dyn;
    int* s_jobs = s_dyn + dm.cap;
    int* s_rev = s_dyn + 2 * dm.cap;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bi = blockIdx.x, kvh = blockIdx.y;
    const int seq = cs.ids[bi];
    const size_t sl = sl_index(dm, seq, layer);
    const int ci = tid % D, sv = tid / D;  // component, vector slot
    const size_t rb = ring_base(dm, seq, layer, kvh);
    const int n_new = cs.n_new[bi];
    // Every load that does not depend on the FIFO step is in flight at once
    // (all are issued before the first LDS store, which would wait for them):
    // metadata, ring tags, row ci of Pi (into registers), S (staged in LDS),
    // and the input tokens (all of them stay hot: an append of at most W
    // tokens evicts only ring entries).
    // S goes straight to LDS (16 bytes per lane); row r's 16-byte block c
    // sits at slot c ^ (r % NB), so that lanes reading the same block of
    // different rows hit different banks.
    static_assert((M * D / 4) % NT == 0, "whole rounds of 16-byte copies");
    // row ci of Pi = column ci of Pi^T: the lanes read consecutive words
    float4 prow[D / 4];
#pragma unroll
    for (int j = 0; j < D / 4; ++j)
        prow[j] = make_float4(P.pit32[(size_t)(4 * j) * D + ci], P.pit32[(size_t)(4 * j + 1) * D + ci],
                              P.pit32[(size_t)(4 * j + 2) * D + ci], P.pit32[(size_t)(4 * j + 3) * D + ci]);
    {
        const float4* gs = reinterpret_cast<const float4*>(P.s32);
        auto copy = [&](const float4* g, float* lds, int nblk) {
            for (int q = 0; q < nblk / NT; ++q) {
                const int pos = q * NT + tid, r = pos / NB, c = pos % NB;
                __builtin_amdgcn_global_load_lds(
                    g + r * NB + (c ^ (r & (NB - 1))),
                    (__attribute__((address_space(3))) void*)(lds + 4 * (q * NT + 64 * wave)), 16, 0, 0);
            }
        };
        copy(gs, &s_s[0][0], M * NB);
    }
    constexpr int TR = 4;  // ring tags per thread in the first round
    const int* gt = P.tags + sl * dm.cap;
    int t4[TR];
#pragma unroll
    for (int r = 0; r < TR; ++r) t4[r] = gt[min(r * NT + tid, dm.cap - 1)];
    static_assert(sizeof(SeqLayerMeta) == 32, "metadata = two 16-byte loads");
    const uint4 meta0 = reinterpret_cast<const uint4*>(P.meta + sl)[0];
    const uint4 meta1 = reinterpret_cast<const uint4*>(P.meta + sl)[1];
    const float cs_t = (tid & 16) ? F.sin_t[tid & 15] : F.cos_t[tid & 15];
    constexpr int KT = SMALL_APPEND_MAX * D / NT;  // kept-token components per thread
    _Float16 kk[KT], kvv[KT];
    {
        // (the inputs may be absent when no sequence appends a token: then
        // any valid address stands in, and nothing read is used)
        const _Float16* ik = n_new > 0 ? in_k : reinterpret_cast<const _Float16*>(P.pi32);
        const _Float16* iv = n_new > 0 ? in_v : reinterpret_cast<const _Float16*>(P.pi32);
        const int tok0 = n_new > 0 ? cs.in_base[bi] : 0;
#pragma unroll
        for (int r = 0; r < KT; ++r) {
            const int idx = r * NT + tid, tt = max(0, min(idx / D, n_new - 1)), k = idx % D;
            const size_t src = n_new > 0 ? ((size_t)(tok0 + tt) * dm.hkv + kvh) * D + k : 0;
            kk[r] = ik[src];
            kvv[r] = iv[src];
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the first LDS store
    // LDS copies
    if (tid == 0) {
        reinterpret_cast<uint4*>(&s_meta)[0] = meta0;
        reinterpret_cast<uint4*>(&s_meta)[1] = meta1;
    }
    if (tid < 32) ((tid & 16) ? s_sin : s_cos)[tid & 15] = cs_t;
#pragma unroll
    for (int r = 0; r < TR; ++r)
        if (r * NT + tid < dm.cap) s_tags[r * NT + tid] = t4[r];
    for (int i = TR * NT + tid; i < dm.cap; i += NT) s_tags[i] = gt[i];  // rings above TR * NT entries
    __syncthreads();
    if (tid == 0) s_pv = plan_view(dm, s_meta, s_tags, cs, bi, s_jobs, s_rev, 1);
    __syncthreads();
    // This block's reads of the shared state are done (their values are in
    // LDS): count it in now, so that the atomic's round trip overlaps the
    // quantisation; the last block of the sequence commits the step at its
    // end.  No fence: nothing this block wrote is read by the others.
    int prior = 0;
    if (tid == 0) prior = atomicAdd(&P.meta[sl].done, 1);
    const PlanView pv = s_pv;
    const int nvec = 2 * pv.pl.n_ring_new;
    constexpr int TB = theta_bits_of(CB), RB = CB - TB, LR = 1 << RB;
    for (int g0 = 0; g0 < nvec; g0 += VP) {
        const int u = g0 + sv;  // vector u: evicted entry u / 2, K (even) or V (odd)
        const bool act = u < nvec;
        const int kv = u & 1;
        const int phys = act ? s_jobs[u >> 1] : 0;
        // ------------------------------------------------ input vector
        s_x[sv][ci] = !act ? 0.0f
                           : (kv == 0 ? (float)P.ring_k[rb + (size_t)phys * D + ci]
                                      : (float)P.ring_v[rb + (size_t)(phys / 32) * D * 32 + (size_t)ci * 32 +
                                                        vpos(phys % 32)]);
        __syncthreads();
        // ------------------------------------------------------ rotation
        float ya = 0.0f, yb = 0.0f, yc = 0.0f, yd = 0.0f;  // inputs k = 0, 1, 2, 3 mod 4
#pragma unroll
        for (int j = 0; j < D / 4; ++j) {
            const float4 xk = *reinterpret_cast<const float4*>(&s_x[sv][4 * j]);
            ya = fmaf(prow[j].x, xk.x, ya);
            yb = fmaf(prow[j].y, xk.y, yb);
            yc = fmaf(prow[j].z, xk.z, yc);
            yd = fmaf(prow[j].w, xk.w, yd);
        }
        const float y = (ya + yb) + (yc + yd);
        const float yo = __shfl_xor(y, 1, 64);
        const float y0 = (ci & 1) ? yo : y, y1 = (ci & 1) ? y : yo;
        const float rr = sqrtf(y0 * y0 + y1 * y1);
        {
            const float m = wave_max(rr);
            if (lane == 0) s_red[0][wave] = m;
        }
        __syncthreads();
        float Rm = s_red[0][sv * WPV];
#pragma unroll
        for (int w = 1; w < WPV; ++w) Rm = fmaxf(Rm, s_red[0][sv * WPV + w]);
        // --------------------------------------------------------- codes
        const _Float16 R16 = (_Float16)Rm;
        float R = (float)R16;
        if (!(R <= 65504.0f)) {
            if (act && ci == 0) atomicOr(P.err, DEVERR_R_OVERFLOW);
            R = 65504.0f;
        }
        const float inv = R > 0.0f ? (float)(LR - 1) / R : 0.0f;
        const float stepr = R / (float)(LR - 1);
        int a = R > 0.0f ? (int)rintf(rr * inv) : 0;
        a = a > LR - 1 ? LR - 1 : a;
        const int b = angle_code_t<TB>(y0, y1, F.half_c, F.half_s);
        const float rh = (float)a * stepr;
        const float e0 = y0 - rh * s_cos[b], e1 = y1 - rh * s_sin[b];
        s_e[sv][ci] = (ci & 1) ? e1 : e0;
        if ((ci & 1) == 0) s_code[sv][ci >> 1] = (uint32_t)(a | (b << RB));
        {
            const float q = wave_sum((ci & 1) ? 0.0f : e0 * e0 + e1 * e1);
            if (lane == 0) s_red[1][wave] = q;
        }
        __syncthreads();
        float e2 = s_red[1][sv * WPV];
#pragma unroll
        for (int w = 1; w < WPV; ++w) e2 += s_red[1][sv * WPV + w];
        // -------------------------------------------------------- sketch
        float z = 0.0f;
        if (ci < M) {
            float za = 0.0f, zb = 0.0f, zc = 0.0f, zd = 0.0f;
#pragma unroll
            for (int j = 0; j < D / 4; ++j) {
                const float4 sk = *reinterpret_cast<const float4*>(&s_s[ci][4 * (j ^ (ci & (NB - 1)))]);
                const float4 ek = *reinterpret_cast<const float4*>(&s_e[sv][4 * j]);
                za = fmaf(sk.x, ek.x, za);
                zb = fmaf(sk.y, ek.y, zb);
                zc = fmaf(sk.z, ek.z, zc);
                zd = fmaf(sk.w, ek.w, zd);
            }
            z = (za + zb) + (zc + zd);
        }
        const uint64_t sbits = __ballot(ci < M && z >= 0.0f);
        // ------------------------------------------------------- packing
        if (act && ci < 64) {  // the vector's first wave
            const int j = u >> 1;
            const int slot = pv.pl.nc_old + j;
            const int tile = slot / TILE, t = slot % TILE;
            const _Float16 rho16 = (_Float16)sqrtf(e2);
            uint8_t* tb = P.cold + cold_tile_offset(dm, F, seq, kvh, kv, tile);
            uint8_t* meta = tb + TILE * (PB + SB);
            if (kv == 0) {
                // K record: position p holds pair pair_of_pos(p)
                if (lane < PB / 4) {
                    uint32_t w = 0;
                    const int p0 = (32 * lane) / CB, p1 = min((32 * lane + 31) / CB, PAIRS - 1);
                    for (int p = p0; p <= p1; ++p) {
                        const uint32_t c = s_code[sv][pair_of_pos(p, D)];
                        const int off = p * CB - 32 * lane;
                        w |= off >= 0 ? (c << off) : (c >> (-off));
                    }
                    reinterpret_cast<uint32_t*>(tb + t * PB)[lane] = w;
                }
                if (lane < SB / 4)
                    reinterpret_cast<uint32_t*>(tb + TILE * PB + t * SB)[lane] = (uint32_t)(sbits >> (32 * lane));
                if (lane == 0) {
                    *reinterpret_cast<_Float16*>(meta + 2 * t) = R16;
                    *reinterpret_cast<_Float16*>(meta + 2 * TILE + 2 * t) = rho16;
                }
            } else {
                // V: the slot's code in every pair row, its sign bit in every sign plane
                const int bit = vpos(t) * CB;
                if (lane < PAIRS) {
                    const uint32_t code = s_code[sv][lane];
                    uint32_t* row = reinterpret_cast<uint32_t*>(tb + (size_t)lane * 4 * CB);
                    atomicOr(row + (bit >> 5), code << (bit & 31));
                    if ((bit & 31) + CB > 32) atomicOr(row + (bit >> 5) + 1, code >> (32 - (bit & 31)));
                }
                if (lane < M && ((sbits >> lane) & 1u))
                    atomicOr(reinterpret_cast<uint32_t*>(tb + TILE * PB) + lane, 1u << vpos(t));
                if (lane == 0) {
                    *reinterpret_cast<_Float16*>(meta + 2 * t) = R16;
                    *reinterpret_cast<_Float16*>(meta + 2 * TILE + 2 * vpos(t)) = rho16;
                }
            }
        }
        __syncthreads();  // the pass's LDS rows are reused by the next pass
    }
    // the kept tokens of this kv head into its ring
#pragma unroll
    for (int r = 0; r < KT; ++r) {
        const int idx = r * NT + tid, tt = idx / D, k = idx % D;
        if (tt < n_new) {
            const int phys = (pv.pl.ring_pos + tt) % dm.cap;
            P.ring_k[rb + (size_t)phys * D + k] = kk[r];
            P.ring_v[rb + (size_t)(phys / 32) * D * 32 + (size_t)k * 32 + vpos(phys % 32)] = kvv[r];
        }
    }
    if (tid == 0) s_last = prior == (int)gridDim.y - 1;
    __syncthreads();
    if (!s_last) return;
    if (tid < n_new) P.tags[sl * dm.cap + (pv.pl.ring_pos + tid) % dm.cap] = -1;
    if (tid == 0) {
        plan_commit(dm, P, layer, seq, pv, s_rev, 1);
        P.meta[sl].done = 0;
    }
}

template <int D, int CB, int M>
__global__ __launch_bounds__(256) void k_append_small(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs,
                                                     const _Float16* __restrict__ in_k,
                                                     const _Float16* __restrict__ in_v) {
    append_small_body<D, CB, M>(dm, P, F, layer, cs, in_k, in_v);
}

// A small append of layer `layer` (format F; blocks z = 0) beside, in blocks
// z >= 1 of the same launch, work on other state that would otherwise take a
// launch of its own:
//  - z == zp: the deferred promotion of another layer layer_p (format Fp, of
//    the same code width) of the same sequences; each layer has its own
//    metadata, ring, cold region and candidate lists;
//  - z == zq: the query preparation of this layer's attention step (q' = Pi q
//    and S q' into the rotated-query buffer, which neither other body reads
//    or writes), with the block size of the other bodies; it writes the same
//    bits as k_qprep.
// zp and zq are -1 when absent.
template <int D, int CB, int M>
__global__ __launch_bounds__(256) void k_append_step(Dims dm, Ptrs P, LayerFmt F, int layer, LayerFmt Fp,
                                                    int layer_p, int zp, CallSeqs cs,
                                                    const _Float16* __restrict__ in_k,
                                                    const _Float16* __restrict__ in_v, int zq,
                                                    const _Float16* __restrict__ q, float cm) {
    static_assert(PNT == 256, "one block size for every body");
    const int z = blockIdx.z;
    if (z == 0) {
        append_small_body<D, CB, M>(dm, P, F, layer, cs, in_k, in_v);
    } else if (z == zp) {
        promote_body<D, CB>(dm, P, Fp, layer_p, cs);
    } else if (z == zq) {
        extern __shared__ float4 s_qdyn[];  // the append body's dynamic LDS, unused by this block
        float* lds = reinterpret_cast<float*>(s_qdyn);
        switch (dm.g) {
            case 1: qprep_body<D, 1, 256>(dm, P, blockIdx.x, blockIdx.y, q, cm, lds); break;
            case 2: qprep_body<D, 2, 256>(dm, P, blockIdx.x, blockIdx.y, q, cm, lds); break;
            case 4: qprep_body<D, 4, 256>(dm, P, blockIdx.x, blockIdx.y, q, cm, lds); break;
            default: qprep_body<D, 8, 256>(dm, P, blockIdx.x, blockIdx.y, q, cm, lds); break;
        }
    }
}

// Dynamic LDS bytes of a qprep_body block for group width g.
template <int D>
static size_t qprep_lds_bytes(int g) {
    switch (g) {
        case 1: return sizeof(float) * QprepGeom<D, 1>::FLOATS;
        case 2: return sizeof(float) * QprepGeom<D, 2>::FLOATS;
        case 4: return sizeof(float) * QprepGeom<D, 4>::FLOATS;
        default: return sizeof(float) * QprepGeom<D, 8>::FLOATS;
    }
}

// Tensor Cache writes ("Tensor Cache: Eviction-conditioned Associative
// Memory for Transformers", gist.science, section "Metodologia": a pair the
// window evicts is written A <- lambda A + eta (k outer v)).  One block per
// (sequence, kv head); the evicted tokens, oldest first, are the plan's ring
// entries (jobs) and then its input rows that go straight out.  Chunks of C
// <= 32 tokens are written at once, A <- lambda^C A + sum_c eta
// lambda^(C-1-c) k_c v_c^T, which is the C sequential writes reordered (the
// weighted scan).  Thread t holds a CPT-wide piece of one row of A in
// registers for the whole launch; the chunk's keys (scaled by their
// weights) and values pass through LDS as fp32.
template <int D>
__global__ __launch_bounds__(256) void k_tc_write(Dims dm, Ptrs P, int layer, CallSeqs cs,
                                                  const _Float16* __restrict__ in_k,
                                                  const _Float16* __restrict__ in_v) {
    constexpr int NT = 256, TPR = NT / D, CPT = D / TPR;  // threads per row of A, columns per thread
    __shared__ __attribute__((aligned(16))) float s_k[TILE][D];
    __shared__ __attribute__((aligned(16))) float s_v[TILE][D];
    const int bi = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
    const AppendPlan pl = P.plan[bi];
    const int n_src = pl.n_ring_new + pl.e_in;
    if (n_src == 0) return;
    const int seq = cs.ids[bi];
    const size_t rb = ring_base(dm, seq, layer, kvh);
    const int* jobs = P.jobs + (size_t)bi * dm.cap;
    float* A = P.tc_a + (sl_index(dm, seq, layer) * dm.hkv + kvh) * (size_t)D * D;
    const int row = tid / TPR, c0 = (tid % TPR) * CPT;
    float a[CPT];
#pragma unroll
    for (int j = 0; j < CPT; j += 4) {
        const float4 x = *reinterpret_cast<const float4*>(A + (size_t)row * D + c0 + j);
        a[j] = x.x, a[j + 1] = x.y, a[j + 2] = x.z, a[j + 3] = x.w;
    }
    for (int b0 = 0; b0 < n_src; b0 += TILE) {
        const int C = min(TILE, n_src - b0);
        __syncthreads();  // the previous chunk's LDS reads are done
        for (int e = tid; e < C * D; e += NT) {
            const int c = e / D, dim = e % D, t = b0 + c;
            float kx, vx;
            if (t < pl.n_ring_new) {
                const int phys = jobs[t];
                kx = (float)P.ring_k[rb + (size_t)phys * D + dim];
                vx = (float)P.ring_v[rb + (size_t)(phys / TILE) * D * TILE + (size_t)dim * TILE + vpos(phys % TILE)];
            } else {
                const size_t r = ((size_t)(pl.in_base + t - pl.n_ring_new) * dm.hkv + kvh) * D + dim;
                kx = (float)in_k[r];
                vx = (float)in_v[r];
            }
            s_k[c][dim] = kx * (dm.tc_eta * dm.tc_pow[C - 1 - c]);
            s_v[c][dim] = vx;
        }
        __syncthreads();
        const float lc = dm.tc_pow[C];
#pragma unroll
        for (int j = 0; j < CPT; ++j) a[j] *= lc;
        for (int c = 0; c < C; ++c) {
            const float kw = s_k[c][row];
#pragma unroll
            for (int j = 0; j < CPT; j += 4) {
                const float4 vv = *reinterpret_cast<const float4*>(&s_v[c][c0 + j]);
                a[j] = fmaf(kw, vv.x, a[j]);
                a[j + 1] = fmaf(kw, vv.y, a[j + 1]);
                a[j + 2] = fmaf(kw, vv.z, a[j + 2]);
                a[j + 3] = fmaf(kw, vv.w, a[j + 3]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CPT; j += 4)
        *reinterpret_cast<float4*>(A + (size_t)row * D + c0 + j) = float4{a[j], a[j + 1], a[j + 2], a[j + 3]};
}

// Large Tensor Cache writes (a prefill evicting many tokens at once).  The
// n evicted tokens of a (sequence, kv head) are cut into up to TC_SEGS
// segments [s0, s1) of at least TC_SEG_MIN tokens; the n sequential writes
// equal A <- lambda^n A + eta sum_s lambda^(n - s1) S_s with
// S_s = sum_{t in [s0, s1)} lambda^(s1 - 1 - t) k_t v_t^T (the weighted scan
// regrouped by segment).  k_tc_seg computes one S_s per block on MFMA:
// S_s = K^T (W V) over the segment's tokens, 32 tokens per step, with K^T
// (fp16, exact) as the A operand and W V split into fp16 hi + lo * 2^-12 as
// two B operands, so each product is exact to about 2^-22 and sums in fp32.
// k_tc_merge then combines the segments in order.
constexpr int TC_NT = 512;  // k_tc_seg threads: 8 waves, each a 2 x 4 (D 128) or 1 x 2 (D 64) set of 16 x 16 blocks
__device__ __forceinline__ int tc_seg_len(int n) {
    const int per = (n + TC_SEGS - 1) / TC_SEGS;
    return max(TC_SEG_MIN, (per + TILE - 1) / TILE * TILE);
}

template <int D>
__global__ __launch_bounds__(TC_NT) void k_tc_seg(Dims dm, Ptrs P, int layer, CallSeqs cs,
                                                  const _Float16* __restrict__ in_k,
                                                  const _Float16* __restrict__ in_v) {
    constexpr int RS = TILE + 8;   // LDS row stride (halves): 80 bytes, 16-byte aligned rows
    constexpr int NB = D / 16;     // 16-wide blocks of rows (dims i) and of columns (dims j)
    constexpr int RW = NB / 4;     // row blocks per wave: wave w takes rows (w % 4) RW ..
    constexpr int CW = NB / 2;     // column blocks per wave: and columns (w / 4) CW ..
    constexpr int NP = TILE * D / 8;               // 16-byte pieces of a step's K (and of its V)
    constexpr int PER = (NP + TC_NT - 1) / TC_NT;  // pieces per thread and step
    __shared__ __attribute__((aligned(16))) _Float16 s_kt[D][RS];  // K^T of the step's 32 tokens
    __shared__ __attribute__((aligned(16))) _Float16 s_bh[D][RS];  // (W V)^T, fp16 hi
    __shared__ __attribute__((aligned(16))) _Float16 s_bl[D][RS];  // (W V)^T, lo * 2^12
    const int bi = blockIdx.x, kvh = blockIdx.y, sg = blockIdx.z, tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb0 = (wave % 4) * RW, cb0 = (wave / 4) * CW;
    const AppendPlan pl = P.plan[bi];
    const int n_src = pl.n_ring_new + pl.e_in;
    const int len = tc_seg_len(n_src);
    const int s0 = sg * len, s1 = min(n_src, s0 + len);
    if (s0 >= s1) return;
    const int seq = cs.ids[bi];
    const size_t rb = ring_base(dm, seq, layer, kvh);
    const int* jobs = P.jobs + (size_t)bi * dm.cap;
    floatx4 ah[RW][CW], al[RW][CW];
#pragma unroll
    for (int a = 0; a < RW; ++a)
#pragma unroll
        for (int b = 0; b < CW; ++b) ah[a][b] = al[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
    // piece e -> token e % 32 of a step, dims 8 (e / 32) .. + 7 (the 32
    // lanes that write one transposed LDS row hold consecutive tokens: no
    // bank conflicts); a step's rows are loaded one step ahead (registers),
    // so the loads of step c0 + 32 are in flight during step c0's MFMAs
    auto load = [&](int c0, uint4 (&kq)[PER], uint4 (&vq)[PER]) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + TC_NT * u, c = e % TILE, d0 = 8 * (e / TILE), t = c0 + c;
            kq[u] = vq[u] = uint4{0u, 0u, 0u, 0u};
            if (e < NP && t < s1) {
                if (t < pl.n_ring_new) {
                    const int phys = jobs[t];
                    kq[u] = *reinterpret_cast<const uint4*>(P.ring_k + rb + (size_t)phys * D + d0);
                    _Float16 vv[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        vv[r] = P.ring_v[rb + (size_t)(phys / TILE) * D * TILE + (size_t)(d0 + r) * TILE +
                                         vpos(phys % TILE)];
                    vq[u] = *reinterpret_cast<const uint4*>(vv);
                } else {
                    const size_t r = ((size_t)(pl.in_base + t - pl.n_ring_new) * dm.hkv + kvh) * D + d0;
                    kq[u] = *reinterpret_cast<const uint4*>(in_k + r);
                    vq[u] = *reinterpret_cast<const uint4*>(in_v + r);
                }
            }
        }
    };
    uint4 kn[PER], vn[PER];
    load(s0, kn, vn);
    const int kq8 = 8 * (lane >> 4), rr = lane & 15;  // operand lane: row / column rr, tokens kq8 .. + 7
    for (int c0 = s0; c0 < s1; c0 += TILE) {
        uint4 kq[PER], vq[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) kq[u] = kn[u], vq[u] = vn[u];
        if (c0 + TILE < s1) load(c0 + TILE, kn, vn);
        __syncthreads();  // the previous step's operand reads are done
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + TC_NT * u, c = e % TILE, d0 = 8 * (e / TILE), t = c0 + c;
            if (e < NP) {
                const float w = t < s1 ? exp2f((float)(s1 - 1 - t) * dm.tc_log2l) : 0.0f;
                const _Float16* kh = reinterpret_cast<const _Float16*>(&kq[u]);
                const _Float16* vh = reinterpret_cast<const _Float16*>(&vq[u]);
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const float x = w * (float)vh[r];
                    const _Float16 hi = (_Float16)x;
                    s_kt[d0 + r][c] = kh[r];
                    s_bh[d0 + r][c] = hi;
                    s_bl[d0 + r][c] = (_Float16)((x - (float)hi) * LO_SCALE);
                }
            }
        }
        __syncthreads();
        half8 bh[CW], bl[CW];
#pragma unroll
        for (int b = 0; b < CW; ++b) {
            bh[b] = *reinterpret_cast<const half8*>(&s_bh[16 * (cb0 + b) + rr][kq8]);
            bl[b] = *reinterpret_cast<const half8*>(&s_bl[16 * (cb0 + b) + rr][kq8]);
        }
#pragma unroll
        for (int a = 0; a < RW; ++a) {
            const half8 ak = *reinterpret_cast<const half8*>(&s_kt[16 * (rb0 + a) + rr][kq8]);
#pragma unroll
            for (int b = 0; b < CW; ++b) {
                ah[a][b] = mfma16x16x32(ak, bh[b], ah[a][b]);
                al[a][b] = mfma16x16x32(ak, bl[b], al[a][b]);
            }
        }
    }
    // S_s[i][j]: lane holds rows 4 (lane / 16) + r, column lane % 16 of each 16 x 16 block
    float* S = P.tc_seg + (((size_t)bi * dm.hkv + kvh) * TC_SEGS + sg) * D * D;
#pragma unroll
    for (int a = 0; a < RW; ++a)
#pragma unroll
        for (int b = 0; b < CW; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * (rb0 + a) + 4 * (lane >> 4) + r, j = 16 * (cb0 + b) + (lane & 15);
                S[(size_t)i * D + j] = ah[a][b][r] + al[a][b][r] * (1.0f / LO_SCALE);
            }
}

// A <- lambda^n A + eta sum_s lambda^(n - s1_s) S_s, segments in order; block
// (sequence, kv head, 16-row slice of A).
template <int D>
__global__ __launch_bounds__(256) void k_tc_merge(Dims dm, Ptrs P, int layer, CallSeqs cs) {
    const int bi = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
    const AppendPlan pl = P.plan[bi];
    const int n_src = pl.n_ring_new + pl.e_in;
    if (n_src == 0) return;
    const int len = tc_seg_len(n_src), nseg = (n_src + len - 1) / len;
    const int seq = cs.ids[bi];
    float* A = P.tc_a + (sl_index(dm, seq, layer) * dm.hkv + kvh) * (size_t)D * D;
    const float* S = P.tc_seg + ((size_t)bi * dm.hkv + kvh) * TC_SEGS * D * D;
    const float ln = exp2f((float)n_src * dm.tc_log2l);
    for (int e = blockIdx.z * 16 * D + tid; e < (blockIdx.z + 1) * 16 * D; e += 256) {
        float acc = 0.0f;
        for (int s = 0; s < nseg; ++s) {
            const int s1 = min(n_src, (s + 1) * len);
            acc = fmaf(exp2f((float)(n_src - s1) * dm.tc_log2l), S[(size_t)s * D * D + e], acc);
        }
        A[e] = fmaf(ln, A[e], dm.tc_eta * acc);
    }
}

hipError_t launch_tc_write(const Dims& dm, const Ptrs& P, int layer, const CallSeqs& cs, int max_new,
                           const _Float16* k, const _Float16* v, hipStream_t st) {
    const dim3 g(cs.n, dm.hkv);
    if (max_new >= TC_SEG_MIN) {
        const dim3 gs(cs.n, dm.hkv, TC_SEGS), gm(cs.n, dm.hkv, dm.d / 16);
        if (dm.d == 64) {
            k_tc_seg<64><<<gs, TC_NT, 0, st>>>(dm, P, layer, cs, k, v);
            k_tc_merge<64><<<gm, 256, 0, st>>>(dm, P, layer, cs);
        } else {
            k_tc_seg<128><<<gs, TC_NT, 0, st>>>(dm, P, layer, cs, k, v);
            k_tc_merge<128><<<gm, 256, 0, st>>>(dm, P, layer, cs);
        }
        return hipGetLastError();
    }
    if (dm.d == 64)
        k_tc_write<64><<<g, 256, 0, st>>>(dm, P, layer, cs, k, v);
    else
        k_tc_write<128><<<g, 256, 0, st>>>(dm, P, layer, cs, k, v);
    return hipGetLastError();
}

// False when the block's LDS (static plus 3 ints per ring slot, or the query
// preparation's share) would not fit: the caller then takes the general path.
// layer_p >= 0: the launch also runs the promotion of layer layer_p (format
// Fp) for the same sequences; q != nullptr: it also prepares the queries of
// this layer's attention step (scale cm of the sketch part).
template <int D, int CB, int M>
static bool small_launch(hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                         const CallSeqs& cs, const _Float16* k, const _Float16* v, const LayerFmt* Fp,
                         int layer_p, const _Float16* q, float cm) {
    static size_t static_lds[2] = {0, 0}, max_lds = 0;
    const int fz = (layer_p >= 0 || q) ? 1 : 0;
    if (static_lds[fz] == 0) {
        hipFuncAttributes fa{};
        int dev = 0, mx = 0;
        const void* fn = fz ? reinterpret_cast<const void*>(k_append_step<D, CB, M>)
                            : reinterpret_cast<const void*>(k_append_small<D, CB, M>);
        if (hipFuncGetAttributes(&fa, fn) != hipSuccess || hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&mx, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return false;
        static_lds[fz] = fa.sharedSizeBytes;
        max_lds = (size_t)mx;
    }
    size_t dyn = (size_t)3 * dm.cap * sizeof(int);
    if (q) dyn = std::max(dyn, qprep_lds_bytes<D>(dm.g));
    if (static_lds[fz] + dyn > max_lds) return false;
    if (fz) {
        int nz = 1;
        const int zp = layer_p >= 0 ? nz++ : -1;
        const int zq = q ? nz++ : -1;
        k_append_step<D, CB, M><<<dim3(cs.n, dm.hkv, nz), 256, dyn, st>>>(
            dm, P, F, layer, Fp ? *Fp : F, layer_p, zp, cs, k, v, zq, q, cm);
    } else {
        k_append_small<D, CB, M><<<dim3(cs.n, dm.hkv), 256, dyn, st>>>(dm, P, F, layer, cs, k, v);
    }
    return true;
}

// CUs of the current device
static int cu_count() {
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 256;
        n_cu = n;
    }
    return n_cu;
}

// items: an upper bound of the launch's items; the grid holds no more blocks
// than are resident at once
template <int D, int CB, int M>
static void quantize_launch(long items, hipStream_t st, const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer,
                            const CallSeqs& cs, const _Float16* k, const _Float16* v) {
    static int resident = 0;
    if (resident == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_quantize<D, CB, M>, QNT, 0) != hipSuccess || nb < 1)
            nb = 1;
        resident = nb * cu_count();
    }
    const long blocks = std::max<long>(1, std::min<long>((items + QNT / 64 - 1) / (QNT / 64), resident));
    k_quantize<D, CB, M><<<(unsigned)blocks, QNT, 0, st>>>(dm, P, F, layer, cs, k, v);
}

// The general path: FIFO plan, then the quantiser over the (cold tile,
// sequence, kv head, K or V) items, then the ring copy of the kept tokens.
static hipError_t append_large(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs,
                               int max_new, const _Float16* k, const _Float16* v, hipStream_t st) {
    const int key = dm.d * 1000 + F.cb * 100 + F.m;
    k_append_plan<<<cs.n, 64, 0, st>>>(dm, P, layer, cs);
    if (dm.tc) {
        // evicted tokens go into the tensor-cache matrices instead of codes
        hipError_t e = launch_tc_write(dm, P, layer, cs, max_new, k, v, st);
        if (e != hipSuccess) return e;
        if (max_new > 0) {
            const dim3 g2((std::min(max_new, dm.W) + TILE - 1) / TILE, cs.n, dm.hkv);
            if (dm.d == 64)
                k_hot_append<64><<<g2, 256, 0, st>>>(dm, P, layer, cs, k, v);
            else
                k_hot_append<128><<<g2, 256, 0, st>>>(dm, P, layer, cs, k, v);
        }
        return hipGetLastError();
    }
    // an upper bound of the items: tiles touched x kv heads x (K, V)
    const long grid = ((long)(max_new + dm.cap) / TILE + 2) * cs.n * dm.hkv * 2;
    switch (key) {
        case 64 * 1000 + 5 * 100 + 32: quantize_launch<64, 5, 32>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 64 * 1000 + 5 * 100 + 64: quantize_launch<64, 5, 64>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 64 * 1000 + 7 * 100 + 32: quantize_launch<64, 7, 32>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 64 * 1000 + 7 * 100 + 64: quantize_launch<64, 7, 64>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 64 * 1000 + 4 * 100 + 32: quantize_launch<64, 4, 32>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 64 * 1000 + 4 * 100 + 64: quantize_launch<64, 4, 64>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 128 * 1000 + 5 * 100 + 32: quantize_launch<128, 5, 32>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 128 * 1000 + 5 * 100 + 64: quantize_launch<128, 5, 64>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 128 * 1000 + 7 * 100 + 32: quantize_launch<128, 7, 32>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 128 * 1000 + 7 * 100 + 64: quantize_launch<128, 7, 64>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 128 * 1000 + 4 * 100 + 32: quantize_launch<128, 4, 32>(grid, st, dm, P, F, layer, cs, k, v); break;
        case 128 * 1000 + 4 * 100 + 64: quantize_launch<128, 4, 64>(grid, st, dm, P, F, layer, cs, k, v); break;
        default: return hipErrorInvalidValue;
    }
    if (max_new > 0) {
        const dim3 g2((std::min(max_new, dm.W) + TILE - 1) / TILE, cs.n, dm.hkv);
        if (dm.d == 64)
            k_hot_append<64><<<g2, 256, 0, st>>>(dm, P, layer, cs, k, v);
        else
            k_hot_append<128><<<g2, 256, 0, st>>>(dm, P, layer, cs, k, v);
    }
    return hipGetLastError();
}

hipError_t launch_append(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs, int max_new,
                         const _Float16* k, const _Float16* v, hipStream_t st, const LayerFmt* Fp, int layer_p,
                         bool* fused, const _Float16* q, float cm, bool* q_done) {
    if (fused) *fused = false;
    if (q_done) *q_done = false;
    if (cs.n == 0) return hipSuccess;
    const int key = dm.d * 1000 + F.cb * 100 + F.m;
    if (!dm.tc && max_new <= SMALL_APPEND_MAX && max_new <= dm.W) {
        // 1 launched, 0 the LDS does not fit, -1 unknown format
        auto small = [&](int lp, const _Float16* qq) -> int {
            switch (key) {
#define TQ_SMALL(D_, CB_, M_) \
    case D_ * 1000 + CB_ * 100 + M_: return small_launch<D_, CB_, M_>(st, dm, P, F, layer, cs, k, v, Fp, lp, qq, cm);
                TQ_SMALL(64, 5, 32) TQ_SMALL(64, 5, 64) TQ_SMALL(64, 7, 32) TQ_SMALL(64, 7, 64)
                TQ_SMALL(64, 4, 32) TQ_SMALL(64, 4, 64) TQ_SMALL(128, 5, 32) TQ_SMALL(128, 5, 64)
                TQ_SMALL(128, 7, 32) TQ_SMALL(128, 7, 64) TQ_SMALL(128, 4, 32) TQ_SMALL(128, 4, 64)
#undef TQ_SMALL
                default: return -1;
            }
        };
        const _Float16* qq = (q && q_done) ? q : nullptr;
        const bool with_p = fused && Fp && layer_p >= 0 && Fp->cb == F.cb;
        // the widest merge whose LDS fits: promotion and query preparation,
        // then the promotion alone, then the append alone
        if (with_p || qq) {
            int r = small(with_p ? layer_p : -1, qq);
            if (r == -1) return hipErrorInvalidValue;
            if (r == 0 && with_p && qq) {
                r = small(layer_p, nullptr);
                qq = nullptr;
            }
            if (r == 1) {
                if (fused) *fused = with_p;
                if (q_done) *q_done = qq != nullptr;
                return hipGetLastError();
            }
        }
        const int r = small(-1, nullptr);
        if (r == -1) return hipErrorInvalidValue;
        if (r == 1) return hipGetLastError();
    }
    return append_large(dm, P, F, layer, cs, max_new, k, v, st);
}

// Eviction without new tokens: the general path with the window set to
// target_hot (only the FIFO plan reads the window).
hipError_t launch_evict(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs, int target_hot,
                        hipStream_t st) {
    if (cs.n == 0) return hipSuccess;
    Dims de = dm;
    de.W = target_hot;
    return append_large(de, P, F, layer, cs, 0, nullptr, nullptr, st);
}

}  // namespace tq
