// libtqkv host runtime: the C ABI of include/tqkv.h.
//
// Validates every call on the host, plans the arena, generates the seeded
// rotation and sketch, keeps host mirrors of what it can know without
// synchronising (tokens appended per (seq, layer), attend/promote order), and
// launches the kernels of tq_append.hip, tq_decode.hip and tq_promote.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/tqkv.h"
#include "tq_internal.h"

using namespace tq;

namespace {

thread_local std::string g_last_error;

tq_status fail(tq_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

tq_status hip_fail(hipError_t e, const char* what) {
    return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint64_t kMagic = 0x74716b7663616368ull;  // "tqkvcach"
constexpr uint64_t kDead = 0xdeadull;

// ---------------------------------------------------------------------------
// Seeded parameters: SplitMix64 streams (Steele, Lea, Flood 2014; finaliser
// constants of the published splitmix64.c), Box-Muller normals, Householder
// QR of a Gaussian matrix with R's diagonal made positive (the Haar Q).
// ---------------------------------------------------------------------------
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

std::vector<double> normals(uint64_t seed, int stream, size_t n) {
    const uint64_t s = mix64(seed + (uint64_t)(stream + 1) * kGamma);
    const size_t npair = (n + 1) / 2;
    std::vector<double> out(2 * npair);
    for (size_t i = 0; i < npair; ++i) {
        const uint64_t a = mix64(s + (uint64_t)(2 * i + 1) * kGamma);
        const uint64_t b = mix64(s + (uint64_t)(2 * i + 2) * kGamma);
        const double u1 = (double)(a >> 11) * 0x1.0p-53;
        const double u2 = (double)(b >> 11) * 0x1.0p-53;
        const double rad = std::sqrt(-2.0 * std::log1p(-u1));
        const double ang = 2.0 * M_PI * u2;
        out[2 * i] = rad * std::cos(ang);
        out[2 * i + 1] = rad * std::sin(ang);
    }
    out.resize(n);
    return out;
}

// Randomized Hadamard rotation (the fast alternative to a dense Haar
// rotation): Pi[i][j] = (-1)^popcount(i & j) s_j / sqrt(d), the Sylvester
// matrix (Walsh functions) with column signs s_j = -1 where the top bit of
// output j of SplitMix64 stream 2 is set.  d is a power of two.
std::vector<double> hadamard_rotation(int d, uint64_t seed) {
    const uint64_t s = mix64(seed + (uint64_t)(2 + 1) * kGamma);
    std::vector<double> pi((size_t)d * d);
    const double sc = 1.0 / std::sqrt((double)d);
    for (int j = 0; j < d; ++j) {
        const double sj = (mix64(s + (uint64_t)(j + 1) * kGamma) >> 63) ? -1.0 : 1.0;
        for (int i = 0; i < d; ++i) pi[(size_t)i * d + j] = (__builtin_popcount((unsigned)(i & j)) & 1 ? -sc : sc) * sj;
    }
    return pi;
}

// Pi (row-major, y = Pi x): Q of the QR of the stream-0 Gaussian d x d matrix,
// column k multiplied by the sign of R[k][k].
std::vector<double> haar_rotation(int d, uint64_t seed) {
    std::vector<double> a = normals(seed, 0, (size_t)d * d);
    std::vector<double> vs((size_t)d * d, 0.0);  // reflector k in column k (rows k..d-1)
    std::vector<double> rdiag(d);
    std::vector<double> v(d);
    for (int k = 0; k < d; ++k) {
        double nrm = 0.0;
        for (int i = k; i < d; ++i) nrm += a[(size_t)i * d + k] * a[(size_t)i * d + k];
        nrm = std::sqrt(nrm);
        const double x0 = a[(size_t)k * d + k];
        const double alpha = x0 >= 0.0 ? -nrm : nrm;
        for (int i = k; i < d; ++i) v[i] = a[(size_t)i * d + k];
        v[k] -= alpha;
        double vn = 0.0;
        for (int i = k; i < d; ++i) vn += v[i] * v[i];
        vn = std::sqrt(vn);
        if (vn > 0.0)
            for (int i = k; i < d; ++i) v[i] /= vn;
        for (int j = k; j < d; ++j) {
            double s = 0.0;
            for (int i = k; i < d; ++i) s += v[i] * a[(size_t)i * d + j];
            for (int i = k; i < d; ++i) a[(size_t)i * d + j] -= 2.0 * v[i] * s;
        }
        for (int i = k; i < d; ++i) vs[(size_t)i * d + k] = v[i];
        rdiag[k] = a[(size_t)k * d + k];
    }
    std::vector<double> q((size_t)d * d, 0.0);
    for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
    for (int k = d - 1; k >= 0; --k) {  // Q = H_0 H_1 ... H_{d-1}
        for (int j = 0; j < d; ++j) {
            double s = 0.0;
            for (int i = k; i < d; ++i) s += vs[(size_t)i * d + k] * q[(size_t)i * d + j];
            for (int i = k; i < d; ++i) q[(size_t)i * d + j] -= 2.0 * vs[(size_t)i * d + k] * s;
        }
    }
    for (int k = 0; k < d; ++k) {
        if (rdiag[k] < 0.0)
            for (int i = 0; i < d; ++i) q[(size_t)i * d + k] = -q[(size_t)i * d + k];
    }
    return q;
}

// ---------------------------------------------------------------------------
// Configuration checks and arena plan.
// ---------------------------------------------------------------------------
bool format_built(const tq_format& f) {
    const bool bits = (f.r_bits == 2 && f.theta_bits == 3) || (f.r_bits == 3 && f.theta_bits == 4) ||
                      (f.r_bits == 2 && f.theta_bits == 2);
    return bits && (f.qjl_m == 32 || f.qjl_m == 64);
}

tq_status check_config(const tq_config* cfg) {
    if (!cfg) return fail(TQ_ERR_INVALID_ARG, "config is NULL");
    if (cfg->n_seq_max <= 0 || cfg->n_layers <= 0 || cfg->n_q_heads <= 0 || cfg->n_kv_heads <= 0)
        return fail(TQ_ERR_INVALID_ARG, "n_seq_max, n_layers and head counts must be positive");
    if (cfg->hot_window <= 0 || cfg->max_context <= 0)
        return fail(TQ_ERR_INVALID_ARG, "hot_window and max_context must be positive");
    if (cfg->n_q_heads % cfg->n_kv_heads)
        return fail(TQ_ERR_UNSUPPORTED, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", cfg->n_q_heads,
                    cfg->n_kv_heads);
    const int g = cfg->n_q_heads / cfg->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(TQ_ERR_UNSUPPORTED, "query heads per kv head must be 1, 2, 4 or 8 (got %d)", g);
    if (cfg->head_dim != 64 && cfg->head_dim != 128)
        return fail(TQ_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", cfg->head_dim);
    if (!cfg->layer_formats) return fail(TQ_ERR_INVALID_ARG, "layer_formats is NULL");
    for (int l = 0; l < cfg->n_layers; ++l) {
        const tq_format& f = cfg->layer_formats[l];
        if (!format_built(f))
            return fail(TQ_ERR_UNSUPPORTED, "layer %d format (r=%d, theta=%d, m=%d) is not built", l, f.r_bits,
                        f.theta_bits, f.qjl_m);
    }
    if (!(cfg->promote_threshold > 1.0f) && !(cfg->promote_threshold >= 1.0f / 64.0f))
        return fail(TQ_ERR_INVALID_ARG, "promote_threshold must be > 1 (off) or in [1/64, 1] (got %g)",
                    (double)cfg->promote_threshold);
    if (cfg->sticky < 1 || cfg->sticky > 255) return fail(TQ_ERR_INVALID_ARG, "sticky must be in [1, 255]");
    if (cfg->v_qjl != 0 && cfg->v_qjl != 1) return fail(TQ_ERR_INVALID_ARG, "v_qjl must be 0 or 1");
    if ((int64_t)cfg->max_context > (1 << 24)) return fail(TQ_ERR_UNSUPPORTED, "max_context above 2^24");
    if (cfg->n_kv_heads > ITEMS_MAX) return fail(TQ_ERR_UNSUPPORTED, "n_kv_heads above %d", ITEMS_MAX);
    if (cfg->rotation_kind != TQ_ROTATION_HAAR && cfg->rotation_kind != TQ_ROTATION_HADAMARD)
        return fail(TQ_ERR_INVALID_ARG, "rotation_kind must be TQ_ROTATION_HAAR or TQ_ROTATION_HADAMARD");
    if (cfg->cold_tier != TQ_COLD_CODES && cfg->cold_tier != TQ_COLD_TENSOR_CACHE)
        return fail(TQ_ERR_INVALID_ARG, "cold_tier must be TQ_COLD_CODES or TQ_COLD_TENSOR_CACHE");
    if (cfg->cold_tier == TQ_COLD_TENSOR_CACHE) {
        if (cfg->promote_threshold <= 1.0f)
            return fail(TQ_ERR_INVALID_ARG, "the tensor-cache tier keeps no cold tokens to promote: "
                                            "promote_threshold must be > 1");
        if (!(cfg->tc_lambda > 0.0f && cfg->tc_lambda <= 1.0f))
            return fail(TQ_ERR_INVALID_ARG, "tc_lambda must be in (0, 1]");
        if (!std::isfinite(cfg->tc_eta)) return fail(TQ_ERR_INVALID_ARG, "tc_eta must be finite");
        if (std::isnan(cfg->tc_gate)) return fail(TQ_ERR_INVALID_ARG, "tc_gate is NaN");
    }
    if (cfg->promote_threshold <= 1.0f &&
        (int64_t)cfg->n_q_heads * (int64_t)std::floor(1.0f / cfg->promote_threshold) > 2048)
        return fail(TQ_ERR_UNSUPPORTED, "n_q_heads * floor(1 / promote_threshold) above 2048");
    return TQ_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    Dims dm;
    std::vector<LayerFmt> fmts;
    size_t o_pi32, o_s32, o_pi_hi, o_pi_lo, o_s_hi, o_s_lo, o_tpi_hi, o_tpi_lo, o_ts_hi, o_ts_lo, o_pit32, o_st32, o_sp32, o_err, o_meta, o_tags, o_tomb, o_sticky, o_cand,
        o_cand_n, o_ring_k, o_ring_v, o_cold, o_tables, o_qprep, o_part, o_cand_chunk, o_plan, o_jobs, o_gate, o_tc,
        o_tc_seg, total;
    size_t clear_bytes;  // bytes from o_err that create() clears (to the end)
};

// Unit pair values of a format, (x, y) = (a / (L_r - 1)) (cos, sin)(phi_b),
// as the tables compute them (fp32).
static void unit_values(int rb, const float* cos_t, const float* sin_t, int tb, std::vector<float>& ux,
                        std::vector<float>& uy) {
    const int ncode = 1 << (rb + tb), LR = 1 << rb;
    ux.resize(ncode);
    uy.resize(ncode);
    for (int code = 0; code < ncode; ++code) {
        const int a = code & (LR - 1), b = code >> rb;
        const float s = (float)a / (float)(LR - 1);
        ux[code] = s * cos_t[b];
        uy[code] = s * sin_t[b];
    }
}

// The value tables hold fp16(S u) and the combine multiplies the value sums
// by 1 / S.  The unit values of a format are a few fixed numbers, so a scale
// S in [1, 2) can be chosen under which all of them lie close to fp16 grid
// points: the largest rounding error max |fp16(S u) - S u| / S over the
// format's values, searched over S = 1 + i / 2^16, falls from about 2^-12
// (S = 1) to about 1e-16 for 2 + 2 bits, 1e-6 for 2 + 3 bits and 7e-5 for
// 3 + 4 bits.  An output's error from the value tables is at most the
// largest value radius R times this.  Ties keep the smallest S.
static float value_scale(int rb, int tb, const float* cos_t, const float* sin_t) {
    static std::mutex mu;
    static std::map<int, float> memo;  // by (rb, tb)
    const int key = rb * 16 + tb;
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = memo.find(key);
        if (it != memo.end()) return it->second;
    }
    std::vector<float> ux, uy;
    unit_values(rb, cos_t, sin_t, tb, ux, uy);
    std::vector<float> u;
    for (size_t i = 0; i < ux.size(); ++i) {
        u.push_back(std::fabs(ux[i]));
        u.push_back(std::fabs(uy[i]));
    }
    std::sort(u.begin(), u.end());
    u.erase(std::unique(u.begin(), u.end()), u.end());
    float best_s = 1.0f;
    double best_e = INFINITY;
    for (int i = 0; i < (1 << 16); ++i) {
        const float sc = 1.0f + (float)i / 65536.0f;
        double e = 0.0;
        for (float v : u) {
            const float x = sc * v;
            e = std::max(e, std::fabs((double)(float)(_Float16)x - (double)x) / (double)sc);
            if (e >= best_e) break;
        }
        if (e < best_e) {
            best_e = e;
            best_s = sc;
        }
    }
    std::lock_guard<std::mutex> lk(mu);
    memo[key] = best_s;
    return best_s;
}

Plan make_plan(const tq_config* cfg) {
    Plan p{};
    Dims& dm = p.dm;
    dm.n_seq_max = cfg->n_seq_max;
    dm.n_layers = cfg->n_layers;
    dm.hq = cfg->n_q_heads;
    dm.hkv = cfg->n_kv_heads;
    dm.d = cfg->head_dim;
    dm.g = dm.hq / dm.hkv;
    dm.W = cfg->hot_window;
    dm.tau = cfg->promote_threshold;
    dm.sticky = cfg->sticky;
    dm.v_qjl = cfg->v_qjl;
    dm.gate = INFINITY;
    dm.mq_n = dm.mq_g = dm.mq_v0 = 0;
    dm.tc = cfg->cold_tier == TQ_COLD_TENSOR_CACHE;
    dm.tc_eta = dm.tc ? cfg->tc_eta : 0.0f;
    // sigmoid(g) without overflow for either sign
    const double gg = dm.tc ? (double)cfg->tc_gate : 0.0;
    dm.tc_sg = (float)(gg >= 0 ? 1.0 / (1.0 + std::exp(-gg)) : std::exp(gg) / (1.0 + std::exp(gg)));
    for (int k = 0; k <= TILE; ++k) dm.tc_pow[k] = dm.tc ? (float)std::pow((double)cfg->tc_lambda, k) : 1.0f;
    dm.tc_log2l = dm.tc ? (float)std::log2((double)cfg->tc_lambda) : 0.0f;
    dm.ktop = dm.tau > 1.0f ? 0 : (int)std::floor(1.0f / dm.tau);
    const int slack = dm.ktop ? dm.hq * dm.ktop : 0;
    dm.cap = (int)(((int64_t)dm.W + slack + TILE - 1) / TILE * TILE);
    // the tensor-cache tier keeps no cold codes: one (unused) tile of slots
    dm.cold_cap = dm.tc ? TILE : (int)(((int64_t)cfg->max_context + TILE - 1) / TILE * TILE);
    dm.max_chunks = ITEMS_MAX;
    dm.call_cap = std::min(dm.n_seq_max, MAX_CALL_SEQ);
    const int d = dm.d;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    p.o_pi32 = take((size_t)d * d * 4);
    p.o_s32 = take((size_t)M_MAX * d * 4);
    p.o_pi_hi = take((size_t)d * d * 2);
    p.o_pi_lo = take((size_t)d * d * 2);
    p.o_s_hi = take((size_t)M_MAX * d * 2);
    p.o_s_lo = take((size_t)M_MAX * d * 2);
    p.o_tpi_hi = take((size_t)3 * d * d * 2);
    p.o_tpi_lo = take((size_t)3 * d * d * 2);
    p.o_ts_hi = take((size_t)3 * M_MAX * d * 2);
    p.o_ts_lo = take((size_t)3 * M_MAX * d * 2);
    p.o_pit32 = take((size_t)d * d * 4);
    p.o_st32 = take((size_t)d * M_MAX * 4);
    p.o_sp32 = take((size_t)M_MAX * d * 4);
    p.o_err = take(16);
    const size_t nsl = (size_t)dm.n_seq_max * dm.n_layers;
    p.o_meta = take(nsl * sizeof(SeqLayerMeta));
    p.o_tags = take(nsl * dm.cap * 4);
    p.o_tomb = take(nsl * (dm.cold_cap / 32) * 4);
    p.o_sticky = take(nsl * dm.cold_cap * 4);
    p.o_cand = take(nsl * dm.hq * std::max(dm.ktop, 1) * sizeof(Cand));
    p.o_cand_n = take(nsl * dm.hq * 4);
    p.o_ring_k = take(nsl * dm.hkv * dm.cap * d * 2);
    p.o_ring_v = take(nsl * dm.hkv * dm.cap * d * 2);
    p.o_cold = o;
    size_t cold = 0, tabs = 0;
    for (int l = 0; l < dm.n_layers; ++l) {
        const tq_format& tf = cfg->layer_formats[l];
        LayerFmt f{};
        f.rb = tf.r_bits;
        f.tb = tf.theta_bits;
        f.m = tf.qjl_m;
        f.cb = f.rb + f.tb;
        f.pb = (d / 2) * f.cb / 8;
        f.sb = f.m / 8;
        f.tile_bytes = TILE * (f.pb + f.sb + 4);
        f.off = cold;
        f.pair2 = f.cb <= 5;
        f.tab_off = tabs;
        // whole KB: the decode kernel stages the tables 1 KB per DMA instruction
        tabs += tables_bytes_of(f.cb);
        const int L = 1 << f.tb;
        for (int b = 0; b < 16; ++b) {
            const double th = -M_PI + 2.0 * M_PI * (double)(b % L) / (double)L;
            f.cos_t[b] = (float)std::cos(th);
            f.sin_t[b] = (float)std::sin(th);
        }
        f.vscale = value_scale(f.rb, f.tb, f.cos_t, f.sin_t);
        f.vscale_inv = 1.0f / f.vscale;
        f.half_c = (float)std::cos(M_PI / (double)L);
        f.half_s = (float)std::sin(M_PI / (double)L);
        for (int b = 0; b < 16; ++b) {
            const double th = -M_PI + 2.0 * M_PI * ((double)(b % L) + 0.5) / (double)L;
            f.cos_h[b] = (float)std::cos(th);
            f.sin_h[b] = (float)std::sin(th);
        }
        cold = align256(cold + (size_t)dm.n_seq_max * dm.hkv * 2 * (dm.cold_cap / TILE) * f.tile_bytes);
        p.fmts.push_back(f);
    }
    o = align256(o + cold);
    p.o_tables = take(tabs);
    p.o_qprep = take((size_t)dm.call_cap * dm.hq * (d + M_MAX) * 4);
    p.o_part = take((size_t)dm.max_chunks * 2 * dm.g * part_stride(d) * 4);
    p.o_cand_chunk = take((size_t)dm.max_chunks * dm.g * std::max(dm.ktop, 1) * sizeof(Cand));
    p.o_plan = take((size_t)dm.call_cap * sizeof(AppendPlan));
    p.o_jobs = take((size_t)dm.call_cap * dm.cap * 4);
    p.o_gate = take((size_t)dm.call_cap * dm.hkv * HOT_SLICES * MAX_G * 4);
    p.o_tc = take(dm.tc ? nsl * dm.hkv * (size_t)d * d * 4 : 0);
    p.o_tc_seg = take(dm.tc ? (size_t)dm.call_cap * dm.hkv * TC_SEGS * d * d * 4 : 0);
    p.total = o;
    // everything after the parameters starts at zero (partial records of parts
    // without tokens are summed with weight 0, so they must hold finite values)
    p.clear_bytes = p.total - p.o_err;
    return p;
}

}  // namespace

struct tq_cache {
    uint64_t magic;
    Plan plan;
    Ptrs P;
    uint8_t* arena;
    std::vector<float> h_pi32, h_s32;
    std::vector<_Float16> h_pi_hi, h_pi_lo, h_s_hi, h_s_lo, h_tpi_hi, h_tpi_lo, h_ts_hi, h_ts_lo;
    std::vector<float> h_pit32, h_st32, h_sp32;
    std::vector<uint8_t> h_tables;
    std::vector<int64_t> appended;   // [seq][layer] tokens appended (host mirror)
    int32_t max_context = 0;         // tokens one sequence may ever append
    std::vector<uint8_t> attended;   // [seq][layer] attention since the last promote
    bool profiling = false;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_used = 0;
    // a promotion deferred by tq_promote_deferred: launched by the next call
    // on the handle, inside a small append's launch where it can be
    struct {
        bool active = false;
        int layer = -1;
        CallSeqs cs{};
        hipStream_t st = nullptr;
    } pend;
};

namespace {

tq_status check_handle(const tq_cache* c) {
    if (!c) return fail(TQ_ERR_INVALID_ARG, "cache handle is NULL");
    if (c->magic != kMagic) return fail(TQ_ERR_INVALID_ARG, "cache handle is not live (destroyed or corrupt)");
    return TQ_OK;
}

// Launches a deferred promotion now, on the stream it was issued on.
tq_status flush_pending(tq_cache* c) {
    if (!c->pend.active) return TQ_OK;
    c->pend.active = false;
    const int l = c->pend.layer;
    hipError_t e = launch_promote(c->plan.dm, c->P, c->plan.fmts[l], l, c->pend.cs, c->pend.st);
    if (e != hipSuccess) return hip_fail(e, "deferred promote launch");
    return TQ_OK;
}

tq_status check_seqs(const tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* ids) {
    const Dims& dm = c->plan.dm;
    if (layer < 0 || layer >= dm.n_layers) return fail(TQ_ERR_INVALID_ARG, "layer %d out of range", layer);
    if (n_seq < 0) return fail(TQ_ERR_INVALID_ARG, "n_seq is negative");
    if (n_seq > 0 && !ids) return fail(TQ_ERR_INVALID_ARG, "seq_ids is NULL");
    std::vector<uint8_t> seen(dm.n_seq_max, 0);
    for (int i = 0; i < n_seq; ++i) {
        if (ids[i] < 0 || ids[i] >= dm.n_seq_max) return fail(TQ_ERR_INVALID_ARG, "seq id %d out of range", ids[i]);
        if (seen[ids[i]]) return fail(TQ_ERR_INVALID_ARG, "seq id %d repeated in one call", ids[i]);
        seen[ids[i]] = 1;
    }
    return TQ_OK;
}

template <typename T>
T* at(uint8_t* base, size_t off) {
    return reinterpret_cast<T*>(base + off);
}

tq_status sync_copy(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t st) {
    hipError_t e = hipMemcpyAsync(dst, src, bytes, kind, st);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return TQ_OK;
}

_Float16 to_half(float x) { return (_Float16)x; }

uint16_t half_bits(_Float16 h) {
    uint16_t u;
    std::memcpy(&u, &h, 2);
    return u;
}

// fp16 hi and lo x 2^12 parts of v (exact split: h + l / 2^12 = v to ~2^-22)
void split_hl(float v, uint16_t& hi, uint16_t& lo) {
    const _Float16 h = to_half(v);
    hi = half_bits(h);
    lo = half_bits(to_half((v - (float)h) * LO_SCALE));
}

// Decode tables of one layer format (layout in tq_internal.h).
void build_tables(const LayerFmt& f, uint8_t* dst) {
    const int ncode = 1 << f.cb;
    std::vector<float> ux, uy;
    unit_values(f.rb, f.cos_t, f.sin_t, f.tb, ux, uy);
    auto vh = [&](float u) { return half_bits(to_half(f.vscale * u)); };  // value entries, scaled
    uint16_t* st = reinterpret_cast<uint16_t*>(dst);
    uint16_t* sm = st + 4 * 16;
    for (int nib = 0; nib < 16; ++nib)
        for (int b = 0; b < 4; ++b) {
            st[4 * nib + b] = ((nib >> b) & 1) ? 0x3C00 : 0xBC00;
            sm[4 * nib + b] = ((nib >> b) & 1) ? 0x0000 : 0x8000;
        }
    uint16_t* kh = reinterpret_cast<uint16_t*>(dst + onetab_off_of(f.cb));
    uint16_t* kl = kh + 2 * ncode;
    uint16_t* v1 = kl + 2 * ncode;
    for (int code = 0; code < ncode; ++code) {
        split_hl(ux[code], kh[2 * code], kl[2 * code]);
        split_hl(uy[code], kh[2 * code + 1], kl[2 * code + 1]);
        v1[2 * code] = vh(ux[code]);
        v1[2 * code + 1] = vh(uy[code]);
    }
    uint16_t* hl = reinterpret_cast<uint16_t*>(dst + khl_off_of(f.cb));
    for (int code = 0; code < ncode; ++code) {
        split_hl(ux[code], hl[4 * code], hl[4 * code + 2]);
        split_hl(uy[code], hl[4 * code + 1], hl[4 * code + 3]);
    }
    if (f.cb <= 5) {
        uint16_t* vxy = reinterpret_cast<uint16_t*>(dst + v2tab_off_of(f.cb));
        uint16_t* kt = reinterpret_cast<uint16_t*>(dst + k2tab_off_of(f.cb));
        for (int idx = 0; idx < ncode * ncode; ++idx) {
            const int a = idx & (ncode - 1), b = idx >> f.cb;
            // entry idx: x(a), x(b), y(a), y(b), one 8-byte read
            vxy[4 * idx] = vh(ux[a]);
            vxy[4 * idx + 1] = vh(ux[b]);
            vxy[4 * idx + 2] = vh(uy[a]);
            vxy[4 * idx + 3] = vh(uy[b]);
            uint16_t* e = kt + 8 * idx;
            split_hl(ux[a], e[0], e[4]);
            split_hl(uy[a], e[1], e[5]);
            split_hl(ux[b], e[2], e[6]);
            split_hl(uy[b], e[3], e[7]);
        }
    }
}

}  // namespace

extern "C" {

const char* tq_status_string(tq_status s) {
    switch (s) {
        case TQ_OK: return "ok";
        case TQ_ERR_INVALID_ARG: return "invalid argument";
        case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case TQ_ERR_CAPACITY: return "capacity exceeded";
        case TQ_ERR_STATE: return "call order violated";
        case TQ_ERR_HIP: return "HIP runtime error";
        case TQ_ERR_DEVICE: return "device-side error latched";
        case TQ_ERR_HOST_ALLOC: return "host allocation failed";
    }
    return "unknown status";
}

const char* tq_last_error(void) { return g_last_error.c_str(); }

uint32_t tq_version(void) { return TQKV_VERSION; }

tq_status tq_cache_required_bytes(const tq_config* cfg, size_t* arena_bytes) {
    tq_status s = check_config(cfg);
    if (s != TQ_OK) return s;
    if (!arena_bytes) return fail(TQ_ERR_INVALID_ARG, "arena_bytes is NULL");
    *arena_bytes = make_plan(cfg).total;
    return TQ_OK;
}

tq_status tq_cache_create(const tq_config* cfg, void* d_arena, size_t arena_bytes, void* stream, tq_cache** out) {
    tq_status s = check_config(cfg);
    if (s != TQ_OK) return s;
    if (!out) return fail(TQ_ERR_INVALID_ARG, "out is NULL");
    if (!d_arena) return fail(TQ_ERR_INVALID_ARG, "arena is NULL");
    if (((uintptr_t)d_arena) & 255) return fail(TQ_ERR_INVALID_ARG, "arena is not 256-byte aligned");
    Plan plan = make_plan(cfg);
    if (arena_bytes < plan.total)
        return fail(TQ_ERR_INVALID_ARG, "arena has %zu bytes, needs %zu", arena_bytes, plan.total);
    tq_cache* c = new (std::nothrow) tq_cache();
    if (!c) return fail(TQ_ERR_HOST_ALLOC, "handle allocation failed");
    c->plan = plan;
    c->arena = (uint8_t*)d_arena;
    const Dims& dm = plan.dm;
    const int d = dm.d;
    uint8_t* A = c->arena;
    Ptrs& P = c->P;
    P.pi32 = at<float>(A, plan.o_pi32);
    P.s32 = at<float>(A, plan.o_s32);
    P.pi_hi = at<_Float16>(A, plan.o_pi_hi);
    P.pit32 = at<float>(A, plan.o_pit32);
    P.st32 = at<float>(A, plan.o_st32);
    P.sp32 = at<float>(A, plan.o_sp32);
    P.pi_lo = at<_Float16>(A, plan.o_pi_lo);
    P.s_hi = at<_Float16>(A, plan.o_s_hi);
    P.s_lo = at<_Float16>(A, plan.o_s_lo);
    P.tpi_hi = at<_Float16>(A, plan.o_tpi_hi);
    P.tpi_lo = at<_Float16>(A, plan.o_tpi_lo);
    P.ts_hi = at<_Float16>(A, plan.o_ts_hi);
    P.ts_lo = at<_Float16>(A, plan.o_ts_lo);
    P.err = at<int32_t>(A, plan.o_err);
    P.meta = at<SeqLayerMeta>(A, plan.o_meta);
    P.tags = at<int32_t>(A, plan.o_tags);
    P.tomb = at<uint32_t>(A, plan.o_tomb);
    P.sticky = at<uint32_t>(A, plan.o_sticky);
    P.cand = at<Cand>(A, plan.o_cand);
    P.cand_n = at<int32_t>(A, plan.o_cand_n);
    P.ring_k = at<_Float16>(A, plan.o_ring_k);
    P.ring_v = at<_Float16>(A, plan.o_ring_v);
    P.cold = at<uint8_t>(A, plan.o_cold);
    P.tables = at<uint8_t>(A, plan.o_tables);
    P.qprep = at<float>(A, plan.o_qprep);
    P.part = at<float>(A, plan.o_part);
    P.cand_chunk = at<Cand>(A, plan.o_cand_chunk);
    P.plan = at<AppendPlan>(A, plan.o_plan);
    P.jobs = at<int32_t>(A, plan.o_jobs);
    P.gate_max = at<float>(A, plan.o_gate);
    P.tc_a = at<float>(A, plan.o_tc);
    P.tc_seg = at<float>(A, plan.o_tc_seg);

    // parameters, fp64 then fp32 and the fp16 hi/lo splits
    std::vector<double> pi64 = cfg->rotation ? std::vector<double>()
                               : (cfg->rotation_kind == TQ_ROTATION_HADAMARD ? hadamard_rotation(d, cfg->seed)
                                                                             : haar_rotation(d, cfg->seed));
    std::vector<double> s64 = cfg->sketch ? std::vector<double>() : normals(cfg->seed, 1, (size_t)M_MAX * d);
    c->h_pi32.resize((size_t)d * d);
    c->h_s32.resize((size_t)M_MAX * d);
    for (size_t i = 0; i < (size_t)d * d; ++i) c->h_pi32[i] = cfg->rotation ? cfg->rotation[i] : (float)pi64[i];
    for (size_t i = 0; i < (size_t)M_MAX * d; ++i) c->h_s32[i] = cfg->sketch ? cfg->sketch[i] : (float)s64[i];
    c->h_pi_hi.resize((size_t)d * d);
    c->h_pi_lo.resize((size_t)d * d);
    for (size_t i = 0; i < (size_t)d * d; ++i) {
        const float x = c->h_pi32[i];
        const _Float16 hi = to_half(x);
        c->h_pi_hi[i] = hi;
        c->h_pi_lo[i] = to_half((x - (float)hi) * LO_SCALE);
    }
    // S rows with their columns in the MFMA operand order of the quantiser
    auto split_s = [&](const float* s32, _Float16* hi_out, _Float16* lo_out) {
        for (int j = 0; j < M_MAX; ++j) {
            for (int kp = 0; kp < d; ++kp) {
                const int kb = kp / 32, q = (kp % 32) / 8, r = kp % 8;
                const int comp = 16 * (2 * kb + (r >= 4)) + 4 * q + (r & 3);
                const float x = s32[(size_t)j * d + comp];
                const _Float16 hi = to_half(x);
                hi_out[(size_t)j * d + kp] = hi;
                lo_out[(size_t)j * d + kp] = to_half((x - (float)hi) * LO_SCALE);
            }
        }
    };
    c->h_s_hi.resize((size_t)M_MAX * d);
    c->h_s_lo.resize((size_t)M_MAX * d);
    split_s(c->h_s32.data(), c->h_s_hi.data(), c->h_s_lo.data());
    // turned copies for tb = 2, 3, 4 angle bits: T turns each pair (y_2p,
    // y_2p+1) by pi / 2^tb; T Pi and S T^T from fp64 sums of the fp32 entries
    c->h_tpi_hi.resize((size_t)3 * d * d);
    c->h_tpi_lo.resize((size_t)3 * d * d);
    c->h_ts_hi.resize((size_t)3 * M_MAX * d);
    c->h_ts_lo.resize((size_t)3 * M_MAX * d);
    {
        std::vector<float> tpi((size_t)d * d), ts((size_t)M_MAX * d);
        for (int t = 0; t < 3; ++t) {
            const double h = M_PI / (double)(1 << (t + 2)), hc = std::cos(h), hs = std::sin(h);
            for (int p2 = 0; p2 < d; p2 += 2)
                for (int k = 0; k < d; ++k) {
                    const double a = c->h_pi32[(size_t)p2 * d + k], b = c->h_pi32[(size_t)(p2 + 1) * d + k];
                    tpi[(size_t)p2 * d + k] = (float)(hc * a - hs * b);
                    tpi[(size_t)(p2 + 1) * d + k] = (float)(hs * a + hc * b);
                }
            for (int j = 0; j < M_MAX; ++j)
                for (int p2 = 0; p2 < d; p2 += 2) {
                    const double a = c->h_s32[(size_t)j * d + p2], b = c->h_s32[(size_t)j * d + p2 + 1];
                    ts[(size_t)j * d + p2] = (float)(hc * a - hs * b);
                    ts[(size_t)j * d + p2 + 1] = (float)(hs * a + hc * b);
                }
            for (size_t i = 0; i < (size_t)d * d; ++i) {
                const _Float16 hi = to_half(tpi[i]);
                c->h_tpi_hi[(size_t)t * d * d + i] = hi;
                c->h_tpi_lo[(size_t)t * d * d + i] = to_half((tpi[i] - (float)hi) * LO_SCALE);
            }
            split_s(ts.data(), c->h_ts_hi.data() + (size_t)t * M_MAX * d, c->h_ts_lo.data() + (size_t)t * M_MAX * d);
        }
    }
    c->h_pit32.resize((size_t)d * d);
    c->h_st32.resize((size_t)d * M_MAX);
    for (int r = 0; r < d; ++r)
        for (int k = 0; k < d; ++k) c->h_pit32[(size_t)k * d + r] = c->h_pi32[(size_t)r * d + k];
    for (int j = 0; j < M_MAX; ++j)
        for (int k = 0; k < d; ++k) c->h_st32[(size_t)k * M_MAX + j] = c->h_s32[(size_t)j * d + k];
    // S Pi (fp64 sums of the fp32 entries): the QJL back-projection and the
    // rotation of the value output folded into one matrix
    c->h_sp32.resize((size_t)M_MAX * d);
    for (int j = 0; j < M_MAX; ++j)
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += (double)c->h_s32[(size_t)j * d + k] * (double)c->h_pi32[(size_t)k * d + i];
            c->h_sp32[(size_t)j * d + i] = (float)acc;
        }
    // per-layer decode tables
    c->h_tables.assign(plan.o_qprep - plan.o_tables, 0);
    for (int l = 0; l < dm.n_layers; ++l) build_tables(plan.fmts[l], c->h_tables.data() + plan.fmts[l].tab_off);
    c->appended.assign((size_t)dm.n_seq_max * dm.n_layers, 0);
    c->max_context = cfg->max_context;
    c->attended.assign((size_t)dm.n_seq_max * dm.n_layers, 0);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = launch_clear(A + plan.o_err, plan.clear_bytes, st);
    if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "clearing the arena");
    }
    struct {
        void* dst;
        const void* src;
        size_t n;
    } cp[] = {{P.pi32, c->h_pi32.data(), c->h_pi32.size() * 4},   {P.s32, c->h_s32.data(), c->h_s32.size() * 4},
              {P.pi_hi, c->h_pi_hi.data(), c->h_pi_hi.size() * 2}, {P.pi_lo, c->h_pi_lo.data(), c->h_pi_lo.size() * 2},
              {P.s_hi, c->h_s_hi.data(), c->h_s_hi.size() * 2},   {P.s_lo, c->h_s_lo.data(), c->h_s_lo.size() * 2},
              {P.tpi_hi, c->h_tpi_hi.data(), c->h_tpi_hi.size() * 2},
              {P.tpi_lo, c->h_tpi_lo.data(), c->h_tpi_lo.size() * 2},
              {P.ts_hi, c->h_ts_hi.data(), c->h_ts_hi.size() * 2},
              {P.ts_lo, c->h_ts_lo.data(), c->h_ts_lo.size() * 2},
              {P.pit32, c->h_pit32.data(), c->h_pit32.size() * 4}, {P.st32, c->h_st32.data(), c->h_st32.size() * 4},
              {P.sp32, c->h_sp32.data(), c->h_sp32.size() * 4},
              {P.tables, c->h_tables.data(), c->h_tables.size()}};
    for (auto& x : cp) {
        e = hipMemcpyAsync(x.dst, x.src, x.n, hipMemcpyHostToDevice, st);
        if (e != hipSuccess) {
            delete c;
            return hip_fail(e, "copying parameters");
        }
    }
    c->magic = kMagic;
    *out = c;
    return TQ_OK;
}

tq_status tq_cache_destroy(tq_cache* c) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    // a deferred promotion is dropped: nothing can observe the cache any more
    for (hipEvent_t ev : c->ev_pool) hipEventDestroy(ev);
    c->magic = kDead;
    delete c;
    return TQ_OK;
}

tq_status tq_cache_geometry(const tq_cache* c, int32_t* hot_capacity, int32_t* logits_stride) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if (hot_capacity) *hot_capacity = c->plan.dm.cap;
    if (logits_stride) *logits_stride = c->plan.dm.cap + c->plan.dm.cold_cap;
    return TQ_OK;
}

// d_q != NULL (a decode step whose appends and attention form one batch):
// the append launch may also prepare the attention's queries; *q_done says
// whether it did.
static tq_status append_impl(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, const int32_t* n_new,
                             const uint16_t* d_k, const uint16_t* d_v, void* stream, const uint16_t* d_q,
                             bool* q_done) {
    if (q_done) *q_done = false;
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = check_seqs(c, layer, n_seq, seq_ids)) != TQ_OK) return s;
    if (n_seq > 0 && !n_new) return fail(TQ_ERR_INVALID_ARG, "n_new is NULL");
    const Dims& dm = c->plan.dm;
    int64_t total = 0;
    for (int i = 0; i < n_seq; ++i) {
        if (n_new[i] < 0) return fail(TQ_ERR_INVALID_ARG, "n_new[%d] is negative", i);
        const int64_t a = c->appended[sl_index(dm, seq_ids[i], layer)];
        if (a + n_new[i] > c->max_context)
            return fail(TQ_ERR_CAPACITY, "sequence %d layer %d would hold %lld tokens, max_context allows %d",
                        seq_ids[i], layer, (long long)(a + n_new[i]), c->max_context);
        total += n_new[i];
    }
    if (total > 0 && (!d_k || !d_v)) return fail(TQ_ERR_INVALID_ARG, "d_k or d_v is NULL");
    if ((((uintptr_t)d_k) | ((uintptr_t)d_v)) & 15) return fail(TQ_ERR_INVALID_ARG, "d_k and d_v must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    // A deferred promotion of another layer of exactly these sequences, on
    // this stream and in a format of the same code and sketch widths, runs in
    // this append's launch (the two touch disjoint state); any other is
    // launched first.
    int layer_p = -1;
    if (c->pend.active) {
        const CallSeqs& pc = c->pend.cs;
        const LayerFmt &fp = c->plan.fmts[c->pend.layer], &fa = c->plan.fmts[layer];
        bool same = c->pend.st == st && c->pend.layer != layer && n_seq <= MAX_CALL_SEQ && pc.n == n_seq &&
                    fp.cb == fa.cb && fp.m == fa.m;
        for (int i = 0; same && i < n_seq; ++i) same = pc.ids[i] == seq_ids[i];
        if (same) {
            layer_p = c->pend.layer;
        } else if ((s = flush_pending(c)) != TQ_OK) {
            return s;
        }
    }
    int64_t base = 0;
    for (int b0 = 0; b0 < n_seq; b0 += MAX_CALL_SEQ) {
        CallSeqs cs{};
        cs.n = std::min(MAX_CALL_SEQ, n_seq - b0);
        int max_new = 0;
        int64_t batch_tokens = 0;
        for (int i = 0; i < cs.n; ++i) {
            cs.ids[i] = seq_ids[b0 + i];
            cs.n_new[i] = n_new[b0 + i];
            cs.in_base[i] = (int32_t)batch_tokens;
            batch_tokens += n_new[b0 + i];
            max_new = std::max(max_new, (int)n_new[b0 + i]);
        }
        const size_t row = (size_t)dm.hkv * dm.d;
        const _Float16* k = d_k ? reinterpret_cast<const _Float16*>(d_k) + base * row : nullptr;
        const _Float16* v = d_v ? reinterpret_cast<const _Float16*>(d_v) + base * row : nullptr;
        bool fused = false;
        const bool rider = d_q && q_done && b0 == 0 && n_seq <= MAX_CALL_SEQ;
        hipError_t e = launch_append(dm, c->P, c->plan.fmts[layer], layer, cs, max_new, k, v, st,
                                     layer_p >= 0 ? &c->plan.fmts[layer_p] : nullptr, layer_p, &fused,
                                     rider ? reinterpret_cast<const _Float16*>(d_q) : nullptr,
                                     qjl_query_scale(c->plan.fmts[layer]), rider ? q_done : nullptr);
        if (layer_p >= 0) {
            if (fused) c->pend.active = false;
            if (e != hipSuccess) return hip_fail(e, "append launch");
            tq_status fs = flush_pending(c);  // not merged (a large append): launched beside it
            if (fs != TQ_OK) return fs;
            layer_p = -1;
        }
        if (e != hipSuccess) return hip_fail(e, "append launch");
        // the mirror follows each batch the device has been given, so that it
        // matches the device even when a later batch fails to launch
        for (int i = 0; i < cs.n; ++i) c->appended[sl_index(dm, cs.ids[i], layer)] += cs.n_new[i];
        base += batch_tokens;
    }
    return TQ_OK;
}

tq_status tq_quantize_append(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, const int32_t* n_new,
                             const uint16_t* d_k, const uint16_t* d_v, void* stream) {
    return append_impl(c, layer, n_seq, seq_ids, n_new, d_k, d_v, stream, nullptr, nullptr);
}

tq_status tq_evict(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, int32_t target_hot,
                   void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    if ((s = check_seqs(c, layer, n_seq, seq_ids)) != TQ_OK) return s;
    if (target_hot < 0) return fail(TQ_ERR_INVALID_ARG, "target_hot (%d) is negative", target_hot);
    const Dims& dm = c->plan.dm;
    hipStream_t st = (hipStream_t)stream;
    for (int b0 = 0; b0 < n_seq; b0 += MAX_CALL_SEQ) {
        CallSeqs cs{};
        cs.n = std::min(MAX_CALL_SEQ, n_seq - b0);
        for (int i = 0; i < cs.n; ++i) cs.ids[i] = seq_ids[b0 + i];  // no new tokens
        hipError_t e = launch_evict(dm, c->P, c->plan.fmts[layer], layer, cs, std::min(target_hot, dm.cap), st);
        if (e != hipSuccess) return hip_fail(e, "evict launch");
    }
    return TQ_OK;
}

static tq_status decode_attention_impl(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, const uint16_t* d_q,
                           float* d_out, float* d_logits_dbg, float gate, void* stream, bool q_ready = false) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    if ((s = check_seqs(c, layer, n_seq, seq_ids)) != TQ_OK) return s;
    if (n_seq > 0 && (!d_q || !d_out)) return fail(TQ_ERR_INVALID_ARG, "d_q or d_out is NULL");
    Dims dm = c->plan.dm;
    dm.gate = gate;
    hipStream_t st = (hipStream_t)stream;
    const int stride = dm.cap + dm.cold_cap;
    // every (sequence, kv head) stream takes at least one split-context part,
    // so a batch holds at most ITEMS_MAX / n_kv_heads sequences
    const int per_call = std::min(MAX_CALL_SEQ, ITEMS_MAX / dm.hkv);
    for (int b0 = 0; b0 < n_seq; b0 += per_call) {
        CallSeqs cs{};
        cs.n = std::min(per_call, n_seq - b0);
        int64_t app[MAX_CALL_SEQ];
        for (int i = 0; i < cs.n; ++i) {
            cs.ids[i] = seq_ids[b0 + i];
            app[i] = c->appended[sl_index(dm, cs.ids[i], layer)];
        }
        const size_t qoff = (size_t)b0 * dm.hq * dm.d;
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (c->profiling) {
            while (c->ev_pool.size() < c->ev_used + 2) {
                hipEvent_t ev;
                // timing only: no system-scope fence (cache writeback and
                // invalidation) when the event is recorded
                hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableSystemFence);
                if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
                c->ev_pool.push_back(ev);
            }
            e0 = c->ev_pool[c->ev_used];
            e1 = c->ev_pool[c->ev_used + 1];
            c->ev_used += 2;
        }
        hipError_t e = launch_decode(dm, c->P, c->plan.fmts[layer], layer, cs, app,
                                     reinterpret_cast<const _Float16*>(d_q) + qoff, d_out + qoff,
                                     d_logits_dbg ? d_logits_dbg + (size_t)b0 * dm.hq * stride : nullptr, stride, st,
                                     e0, e1, q_ready && b0 == 0);
        if (e != hipSuccess) return hip_fail(e, "decode launch");
    }
    for (int i = 0; i < n_seq; ++i) c->attended[sl_index(dm, seq_ids[i], layer)] = 1;
    return TQ_OK;
}

tq_status tq_decode_attention(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, const uint16_t* d_q,
                              float* d_out, float* d_logits_dbg, void* stream) {
    return decode_attention_impl(c, layer, n_seq, seq_ids, d_q, d_out, d_logits_dbg, INFINITY, stream);
}

tq_status tq_decode_step(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, const int32_t* n_new,
                         const uint16_t* d_k, const uint16_t* d_v, const uint16_t* d_q, float* d_out, void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = check_seqs(c, layer, n_seq, seq_ids)) != TQ_OK) return s;
    if (n_seq > 0 && (!d_q || !d_out)) return fail(TQ_ERR_INVALID_ARG, "d_q or d_out is NULL");
    const Dims& dm = c->plan.dm;
    // the append launch prepares the queries only when the attention runs
    // as one batch (the prepared rows are indexed by the batch position)
    const bool one_batch = n_seq <= std::min(MAX_CALL_SEQ, ITEMS_MAX / dm.hkv);
    bool q_done = false;
    if ((s = append_impl(c, layer, n_seq, seq_ids, n_new, d_k, d_v, stream, one_batch ? d_q : nullptr, &q_done)) !=
        TQ_OK)
        return s;
    return decode_attention_impl(c, layer, n_seq, seq_ids, d_q, d_out, nullptr, INFINITY, stream, q_done);
}

tq_status tq_decode_attention_gated(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids,
                                    const uint16_t* d_q, float* d_out, float* d_logits_dbg, float threshold,
                                    void* stream) {
    if (std::isnan(threshold)) return fail(TQ_ERR_INVALID_ARG, "threshold is NaN");
    return decode_attention_impl(c, layer, n_seq, seq_ids, d_q, d_out, d_logits_dbg, threshold, stream);
}

tq_status tq_decode_attention_static(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids,
                                     const uint16_t* d_q, float* d_out, float* d_logits_dbg, void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    if ((s = check_seqs(c, layer, n_seq, seq_ids)) != TQ_OK) return s;
    if (n_seq > 0 && (!d_q || !d_out)) return fail(TQ_ERR_INVALID_ARG, "d_q or d_out is NULL");
    const Dims& dm = c->plan.dm;
    const int d = dm.d;
    // bytes of the workspace: rotated queries per sequence, partial records
    // and candidates per split-context part
    const size_t q_seq = (size_t)dm.hq * (d + M_MAX) * 4;
    const size_t per_item = (size_t)2 * dm.g * part_stride(d) * 4 + (size_t)dm.g * std::max(dm.ktop, 1) * sizeof(Cand);
    auto fits = [&](int n) { return align256((size_t)n * q_seq) + 512 + (size_t)n * dm.hkv * per_item <= STATIC_WS_BYTES; };
    if (n_seq > 0 && !fits(1))
        return fail(TQ_ERR_CAPACITY,
                    "one sequence needs %zu bytes of decode workspace (%d query heads, %d kv heads, head_dim %d); "
                    "the static workspace holds %zu",
                    align256(q_seq) + 512 + dm.hkv * per_item, dm.hq, dm.hkv, d, STATIC_WS_BYTES);
    int per_call = std::min(MAX_CALL_SEQ, ITEMS_MAX / dm.hkv);
    while (per_call > 1 && !fits(per_call)) --per_call;
    uint8_t* ws = nullptr;
    if (n_seq > 0) {
        hipError_t e = static_workspace(reinterpret_cast<void**>(&ws));
        if (e != hipSuccess) return hip_fail(e, "static workspace address");
    }
    hipStream_t st = (hipStream_t)stream;
    const int stride = dm.cap + dm.cold_cap;
    for (int b0 = 0; b0 < n_seq; b0 += per_call) {
        CallSeqs cs{};
        cs.n = std::min(per_call, n_seq - b0);
        int64_t app[MAX_CALL_SEQ];
        for (int i = 0; i < cs.n; ++i) {
            cs.ids[i] = seq_ids[b0 + i];
            app[i] = c->appended[sl_index(dm, cs.ids[i], layer)];
        }
        // this batch's layout: queries, then as many parts as fit
        const size_t q_bytes = align256((size_t)cs.n * q_seq);
        const size_t items = std::min<size_t>(ITEMS_MAX, (STATIC_WS_BYTES - q_bytes - 512) / per_item);
        const size_t part_bytes = align256(items * 2 * dm.g * part_stride(d) * 4);
        Dims dmb = dm;
        dmb.max_chunks = (int)items;
        Ptrs P = c->P;
        P.qprep = reinterpret_cast<float*>(ws);
        P.part = reinterpret_cast<float*>(ws + q_bytes);
        P.cand_chunk = reinterpret_cast<Cand*>(ws + q_bytes + part_bytes);
        const size_t qoff = (size_t)b0 * dm.hq * d;
        hipError_t e = launch_decode(dmb, P, c->plan.fmts[layer], layer, cs, app,
                                     reinterpret_cast<const _Float16*>(d_q) + qoff, d_out + qoff,
                                     d_logits_dbg ? d_logits_dbg + (size_t)b0 * dm.hq * stride : nullptr, stride, st,
                                     nullptr, nullptr);
        if (e != hipSuccess) return hip_fail(e, "decode launch");
    }
    for (int i = 0; i < n_seq; ++i) c->attended[sl_index(dm, seq_ids[i], layer)] = 1;
    return TQ_OK;
}

tq_status tq_probe_read_bandwidth(const void* d_buf, size_t bytes, uint32_t* d_sink, int32_t blocks, void* stream) {
    if (!d_buf || !d_sink) return fail(TQ_ERR_INVALID_ARG, "d_buf or d_sink is NULL");
    if (bytes == 0 || bytes % 16 || ((uintptr_t)d_buf & 15))
        return fail(TQ_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 and d_buf 16-byte aligned");
    if (blocks < 1 || blocks > (1 << 20)) return fail(TQ_ERR_INVALID_ARG, "blocks out of range");
    hipError_t e = launch_probe_read(d_buf, bytes, d_sink, blocks, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "probe launch");
    return TQ_OK;
}

static tq_status promote_common(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, void* stream,
                                bool defer) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = check_seqs(c, layer, n_seq, seq_ids)) != TQ_OK) return s;
    const Dims& dm = c->plan.dm;
    for (int i = 0; i < n_seq; ++i)
        if (!c->attended[sl_index(dm, seq_ids[i], layer)])
            return fail(TQ_ERR_STATE, "promote on sequence %d layer %d without an attention step since the last one",
                        seq_ids[i], layer);
    if ((s = flush_pending(c)) != TQ_OK) return s;
    for (int i = 0; i < n_seq; ++i) c->attended[sl_index(dm, seq_ids[i], layer)] = 0;
    if (dm.ktop == 0 || n_seq == 0) return TQ_OK;  // promotion disabled
    hipStream_t st = (hipStream_t)stream;
    if (defer && n_seq <= MAX_CALL_SEQ) {
        c->pend.active = true;
        c->pend.layer = layer;
        c->pend.cs = CallSeqs{};
        c->pend.cs.n = n_seq;
        for (int i = 0; i < n_seq; ++i) c->pend.cs.ids[i] = seq_ids[i];
        c->pend.st = st;
        return TQ_OK;
    }
    for (int b0 = 0; b0 < n_seq; b0 += MAX_CALL_SEQ) {
        CallSeqs cs{};
        cs.n = std::min(MAX_CALL_SEQ, n_seq - b0);
        for (int i = 0; i < cs.n; ++i) cs.ids[i] = seq_ids[b0 + i];
        hipError_t e = launch_promote(dm, c->P, c->plan.fmts[layer], layer, cs, st);
        if (e != hipSuccess) return hip_fail(e, "promote launch");
    }
    return TQ_OK;
}

tq_status tq_promote(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, void* stream) {
    return promote_common(c, layer, n_seq, seq_ids, stream, false);
}

tq_status tq_promote_deferred(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, void* stream) {
    return promote_common(c, layer, n_seq, seq_ids, stream, true);
}

tq_status tq_flush(tq_cache* c) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    return flush_pending(c);
}

tq_status tq_cache_sync_stats(tq_cache* c, int32_t seq, int32_t layer, tq_stats* out, void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    const Dims& dm = c->plan.dm;
    if (!out) return fail(TQ_ERR_INVALID_ARG, "out is NULL");
    if (seq < 0 || seq >= dm.n_seq_max || layer < 0 || layer >= dm.n_layers)
        return fail(TQ_ERR_INVALID_ARG, "seq or layer out of range");
    hipStream_t st = (hipStream_t)stream;
    SeqLayerMeta m;
    int32_t err[4];
    if ((s = sync_copy(&m, c->P.meta + sl_index(dm, seq, layer), sizeof(m), hipMemcpyDeviceToHost, st)) != TQ_OK)
        return s;
    if ((s = sync_copy(err, c->P.err, sizeof(err), hipMemcpyDeviceToHost, st)) != TQ_OK) return s;
    std::vector<uint32_t> tomb(dm.cold_cap / 32);
    if ((s = sync_copy(tomb.data(), c->P.tomb + sl_index(dm, seq, layer) * (dm.cold_cap / 32), tomb.size() * 4,
                       hipMemcpyDeviceToHost, st)) != TQ_OK)
        return s;
    int dead = 0;
    for (uint32_t w : tomb) dead += __builtin_popcount(w);
    out->hot_len = m.count;
    out->cold_len = m.cold_len;
    out->live_cold = m.cold_len - dead;
    out->n_promoted = m.n_promoted;
    out->n_evicted = m.n_evicted;
    out->attn_steps = m.attn_step;
    out->device_error = err[0];
    out->hot_capacity = dm.cap;
    out->tokens_appended = c->appended[sl_index(dm, seq, layer)];
    if (err[0]) return fail(TQ_ERR_DEVICE, "device error bits 0x%x latched", err[0]);
    return TQ_OK;
}

namespace {

// Bits [bit, bit + n) of a little-endian byte string (n <= 25).
inline uint32_t get_bits(const uint8_t* p, int bit, int n) {
    uint32_t v = 0;
    for (int i = 0; i < n; ++i) v |= (uint32_t)((p[(bit + i) >> 3] >> ((bit + i) & 7)) & 1u) << i;
    return v;
}

inline void put_bits(uint8_t* p, int bit, int n, uint32_t v) {
    for (int i = 0; i < n; ++i) {
        uint8_t& b = p[(bit + i) >> 3];
        const uint8_t mask = (uint8_t)(1u << ((bit + i) & 7));
        if ((v >> i) & 1u)
            b |= mask;
        else
            b &= (uint8_t)~mask;
    }
}

tq_status codes_common(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, int32_t kv, int32_t first, int32_t n,
                       const void* buf, hipStream_t st, SeqLayerMeta* m) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    const Dims& dm = c->plan.dm;
    if (seq < 0 || seq >= dm.n_seq_max || layer < 0 || layer >= dm.n_layers || kv_head < 0 || kv_head >= dm.hkv ||
        (kv != 0 && kv != 1))
        return fail(TQ_ERR_INVALID_ARG, "seq, layer, kv_head or kv out of range");
    if (first < 0 || n < 0) return fail(TQ_ERR_INVALID_ARG, "negative slot range");
    if (n > 0 && !buf) return fail(TQ_ERR_INVALID_ARG, "host buffer is NULL");
    if ((s = sync_copy(m, c->P.meta + sl_index(dm, seq, layer), sizeof(*m), hipMemcpyDeviceToHost, st)) != TQ_OK)
        return s;
    if ((int64_t)first + n > m->cold_len)
        return fail(TQ_ERR_INVALID_ARG, "slots [%d, %d) beyond the %d written", first, first + n, m->cold_len);
    return TQ_OK;
}

// Convert slot `t` of a device tile image to / from a canonical record.
void tile_to_record(const LayerFmt& f, int d, int kv, const uint8_t* tile, int t, uint8_t* rec) {
    const int P = d / 2, cb = f.cb;
    const int pbc = (P * cb + 7) / 8;
    std::memset(rec, 0, pbc + f.sb + 4);
    for (int i = 0; i < P; ++i) {
        uint32_t code;
        if (kv == 0) {
            int pos = 0;
            for (int p = 0; p < P; ++p)
                if (pair_of_pos(p, d) == i) pos = p;
            code = get_bits(tile + t * f.pb, pos * cb, cb);
        } else {
            code = get_bits(tile + (size_t)i * 4 * cb, vpos(t) * cb, cb);
        }
        put_bits(rec, i * cb, cb, code);
    }
    const uint8_t* sg = tile + TILE * f.pb;
    for (int j = 0; j < f.m; ++j) {
        uint32_t bit = kv == 0 ? get_bits(sg + t * f.sb, j, 1) : get_bits(sg + (size_t)j * 4, vpos(t), 1);
        put_bits(rec + pbc, j, 1, bit);
    }
    const uint8_t* meta = tile + TILE * (f.pb + f.sb);
    std::memcpy(rec + pbc + f.sb, meta + 2 * t, 2);
    std::memcpy(rec + pbc + f.sb + 2, meta + 2 * TILE + 2 * (kv == 0 ? t : vpos(t)), 2);
}

void record_to_tile(const LayerFmt& f, int d, int kv, uint8_t* tile, int t, const uint8_t* rec) {
    const int P = d / 2, cb = f.cb;
    const int pbc = (P * cb + 7) / 8;
    for (int p = 0; p < P; ++p) {
        const int i = pair_of_pos(p, d);
        const uint32_t code = get_bits(rec, i * cb, cb);
        if (kv == 0)
            put_bits(tile + t * f.pb, p * cb, cb, code);
        else
            put_bits(tile + (size_t)i * 4 * cb, vpos(t) * cb, cb, code);
    }
    uint8_t* sg = tile + TILE * f.pb;
    for (int j = 0; j < f.m; ++j) {
        const uint32_t bit = get_bits(rec + pbc, j, 1);
        if (kv == 0)
            put_bits(sg + t * f.sb, j, 1, bit);
        else
            put_bits(sg + (size_t)j * 4, vpos(t), 1, bit);
    }
    uint8_t* meta = tile + TILE * (f.pb + f.sb);
    std::memcpy(meta + 2 * t, rec + pbc + f.sb, 2);
    std::memcpy(meta + 2 * TILE + 2 * (kv == 0 ? t : vpos(t)), rec + pbc + f.sb + 2, 2);
}

}  // namespace

tq_status tq_export_codes(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, int32_t kv, int32_t first_slot,
                          int32_t n, uint8_t* host_out, void* stream) {
    SeqLayerMeta m;
    hipStream_t st = (hipStream_t)stream;
    tq_status s = codes_common(c, seq, layer, kv_head, kv, first_slot, n, host_out, st, &m);
    if (s != TQ_OK || n == 0) return s;
    const Dims& dm = c->plan.dm;
    const LayerFmt& f = c->plan.fmts[layer];
    const int t0 = first_slot / TILE, t1 = (first_slot + n - 1) / TILE;
    // tile pairs t0..t1 (K and V tiles alternate)
    std::vector<uint8_t> img((size_t)(t1 - t0 + 1) * 2 * f.tile_bytes);
    if ((s = sync_copy(img.data(), c->P.cold + cold_tile_offset(dm, f, seq, kv_head, 0, t0), img.size(),
                       hipMemcpyDeviceToHost, st)) != TQ_OK)
        return s;
    const int rb = (dm.d / 2 * f.cb + 7) / 8 + f.sb + 4;
    for (int i = 0; i < n; ++i) {
        const int slot = first_slot + i;
        tile_to_record(f, dm.d, kv, img.data() + ((size_t)(slot / TILE - t0) * 2 + kv) * f.tile_bytes, slot % TILE,
                       host_out + (size_t)i * rb);
    }
    return TQ_OK;
}

tq_status tq_import_codes(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, int32_t kv, int32_t first_slot,
                          int32_t n, const uint8_t* host_in, void* stream) {
    SeqLayerMeta m;
    hipStream_t st = (hipStream_t)stream;
    tq_status s = codes_common(c, seq, layer, kv_head, kv, first_slot, n, host_in, st, &m);
    if (s != TQ_OK || n == 0) return s;
    const Dims& dm = c->plan.dm;
    const LayerFmt& f = c->plan.fmts[layer];
    const int t0 = first_slot / TILE, t1 = (first_slot + n - 1) / TILE;
    std::vector<uint8_t> img((size_t)(t1 - t0 + 1) * 2 * f.tile_bytes);
    uint8_t* dev = c->P.cold + cold_tile_offset(dm, f, seq, kv_head, 0, t0);
    if ((s = sync_copy(img.data(), dev, img.size(), hipMemcpyDeviceToHost, st)) != TQ_OK) return s;
    const int rb = (dm.d / 2 * f.cb + 7) / 8 + f.sb + 4;
    for (int i = 0; i < n; ++i) {
        const int slot = first_slot + i;
        record_to_tile(f, dm.d, kv, img.data() + ((size_t)(slot / TILE - t0) * 2 + kv) * f.tile_bytes, slot % TILE,
                       host_in + (size_t)i * rb);
    }
    return sync_copy(dev, img.data(), img.size(), hipMemcpyHostToDevice, st);
}

tq_status tq_export_hot(tq_cache* c, int32_t seq, int32_t layer, int32_t* n_hot, int32_t* host_tags, uint16_t* host_k,
                        uint16_t* host_v, void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    const Dims& dm = c->plan.dm;
    if (seq < 0 || seq >= dm.n_seq_max || layer < 0 || layer >= dm.n_layers)
        return fail(TQ_ERR_INVALID_ARG, "seq or layer out of range");
    if (!n_hot || !host_tags) return fail(TQ_ERR_INVALID_ARG, "n_hot or host_tags is NULL");
    hipStream_t st = (hipStream_t)stream;
    SeqLayerMeta m;
    const size_t sl = sl_index(dm, seq, layer);
    if ((s = sync_copy(&m, c->P.meta + sl, sizeof(m), hipMemcpyDeviceToHost, st)) != TQ_OK) return s;
    std::vector<int32_t> tags(dm.cap);
    if ((s = sync_copy(tags.data(), c->P.tags + sl * dm.cap, tags.size() * 4, hipMemcpyDeviceToHost, st)) != TQ_OK)
        return s;
    *n_hot = m.count;
    for (int j = 0; j < dm.cap; ++j) host_tags[j] = j < m.count ? tags[(m.head + j) % dm.cap] : -1;
    const size_t per = (size_t)dm.cap * dm.d;
    std::vector<uint16_t> img(per);
    for (int which = 0; which < 2; ++which) {
        uint16_t* dst = which == 0 ? host_k : host_v;
        if (!dst) continue;
        const _Float16* src = which == 0 ? c->P.ring_k : c->P.ring_v;
        for (int h = 0; h < dm.hkv; ++h) {
            if ((s = sync_copy(img.data(), src + ring_base(dm, seq, layer, h), per * 2, hipMemcpyDeviceToHost, st)) !=
                TQ_OK)
                return s;
            uint16_t* o = dst + (size_t)h * per;
            std::memset(o, 0, per * 2);
            for (int j = 0; j < m.count; ++j) {
                const int phys = (m.head + j) % dm.cap;
                for (int k = 0; k < dm.d; ++k)
                    o[(size_t)j * dm.d + k] = which == 0 ? img[(size_t)phys * dm.d + k]
                                                          : img[(size_t)(phys / 32) * dm.d * 32 + k * 32 + vpos(phys % 32)];
            }
        }
    }
    return TQ_OK;
}

tq_status tq_export_paging(tq_cache* c, int32_t seq, int32_t layer, int32_t n, uint8_t* host_live, int32_t* host_sticky,
                           void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    const Dims& dm = c->plan.dm;
    if (seq < 0 || seq >= dm.n_seq_max || layer < 0 || layer >= dm.n_layers || n < 0 || n > dm.cold_cap)
        return fail(TQ_ERR_INVALID_ARG, "seq, layer or n out of range");
    hipStream_t st = (hipStream_t)stream;
    const size_t sl = sl_index(dm, seq, layer);
    SeqLayerMeta m;
    if ((s = sync_copy(&m, c->P.meta + sl, sizeof(m), hipMemcpyDeviceToHost, st)) != TQ_OK) return s;
    std::vector<uint32_t> tomb(dm.cold_cap / 32), stk(dm.cold_cap);
    if ((s = sync_copy(tomb.data(), c->P.tomb + sl * (dm.cold_cap / 32), tomb.size() * 4, hipMemcpyDeviceToHost, st)) !=
        TQ_OK)
        return s;
    if ((s = sync_copy(stk.data(), c->P.sticky + sl * dm.cold_cap, stk.size() * 4, hipMemcpyDeviceToHost, st)) != TQ_OK)
        return s;
    for (int j = 0; j < n; ++j) {
        if (host_live) host_live[j] = ((tomb[j / 32] >> (j % 32)) & 1u) ? 0 : 1;
        if (host_sticky) {
            const uint32_t w = stk[j];
            host_sticky[j] = ((int32_t)(w >> 8) == m.attn_step && m.attn_step > 0) ? (int32_t)(w & 255u) : 0;
        }
    }
    return TQ_OK;
}

tq_status tq_export_tensor_cache(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, float* host_a,
                                 void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    const Dims& dm = c->plan.dm;
    if (!dm.tc) return fail(TQ_ERR_STATE, "the cache keeps codes, not a tensor-cache matrix");
    if (!host_a) return fail(TQ_ERR_INVALID_ARG, "host_a is NULL");
    if (seq < 0 || seq >= dm.n_seq_max || layer < 0 || layer >= dm.n_layers || kv_head < 0 || kv_head >= dm.hkv)
        return fail(TQ_ERR_INVALID_ARG, "seq, layer or kv_head out of range");
    const size_t dd = (size_t)dm.d * dm.d;
    return sync_copy(host_a, c->P.tc_a + (sl_index(dm, seq, layer) * dm.hkv + kv_head) * dd, dd * 4,
                     hipMemcpyDeviceToHost, (hipStream_t)stream);
}

tq_status tq_mips_workspace_bytes(const tq_cache* c, int32_t n_q, int32_t k, size_t* bytes) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if (!bytes) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
    if (n_q < 1 || n_q > TQ_MIPS_MAX_QUERIES) return fail(TQ_ERR_INVALID_ARG, "n_q must be in [1, %d]", TQ_MIPS_MAX_QUERIES);
    if (k < 1 || k > TQ_MIPS_MAX_K) return fail(TQ_ERR_INVALID_ARG, "k must be in [1, %d]", TQ_MIPS_MAX_K);
    // an upper bound over stream lengths (the part count grows with the length up to its cap)
    *bytes = mips_workspace_bytes(c->plan.dm, n_q, k, (int64_t)1 << 40);
    return TQ_OK;
}

tq_status tq_mips_search(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, int32_t n_q, const uint16_t* d_q,
                         int32_t k, int32_t* d_idx, float* d_score, void* d_workspace, size_t workspace_bytes,
                         void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = flush_pending(c)) != TQ_OK) return s;
    const Dims& dm = c->plan.dm;
    if (dm.tc) return fail(TQ_ERR_STATE, "the tensor-cache tier keeps no coded vectors to search");
    if (seq < 0 || seq >= dm.n_seq_max || layer < 0 || layer >= dm.n_layers || kv_head < 0 || kv_head >= dm.hkv)
        return fail(TQ_ERR_INVALID_ARG, "seq, layer or kv_head out of range");
    if (n_q < 1 || n_q > TQ_MIPS_MAX_QUERIES) return fail(TQ_ERR_INVALID_ARG, "n_q must be in [1, %d]", TQ_MIPS_MAX_QUERIES);
    if (k < 1 || k > TQ_MIPS_MAX_K) return fail(TQ_ERR_INVALID_ARG, "k must be in [1, %d]", TQ_MIPS_MAX_K);
    if (!d_q || !d_idx || !d_score || !d_workspace) return fail(TQ_ERR_INVALID_ARG, "a pointer is NULL");
    if ((uintptr_t)d_workspace & 255) return fail(TQ_ERR_INVALID_ARG, "d_workspace must be 256-byte aligned");
    const int64_t app = c->appended[sl_index(dm, seq, layer)];
    const size_t need = mips_workspace_bytes(dm, n_q, k, app);
    if (workspace_bytes < need)
        return fail(TQ_ERR_INVALID_ARG, "workspace of %zu bytes, the search needs %zu", workspace_bytes, need);
    hipError_t e = launch_mips(dm, c->P, c->plan.fmts[layer], layer, seq, kv_head, n_q,
                               reinterpret_cast<const _Float16*>(d_q), k, d_idx, d_score,
                               reinterpret_cast<uint8_t*>(d_workspace), app, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "search launch");
    return TQ_OK;
}

tq_status tq_multi_query_workspace_bytes(const tq_cache* c, size_t* bytes) {
    return tq_multi_query_batch_workspace_bytes(c, 1, bytes);
}

tq_status tq_multi_query_batch_workspace_bytes(const tq_cache* c, int32_t n_seq, size_t* bytes) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if (!bytes) return fail(TQ_ERR_INVALID_ARG, "bytes is NULL");
    if (n_seq < 1 || n_seq > std::min(MAX_CALL_SEQ, MQ_STREAMS_MAX / c->plan.dm.hkv))
        return fail(TQ_ERR_INVALID_ARG, "n_seq (%d) must be in [1, %d]", n_seq,
                    std::min(MAX_CALL_SEQ, MQ_STREAMS_MAX / c->plan.dm.hkv));
    *bytes = multi_query_workspace_bytes(c->plan.dm, n_seq);
    return TQ_OK;
}

tq_status tq_multi_query_attention(tq_cache* c, int32_t layer, int32_t seq, int32_t n_new, const uint16_t* d_q,
                                   float* d_out, void* d_workspace, size_t workspace_bytes, void* stream) {
    return tq_multi_query_attention_batch(c, layer, 1, &seq, n_new, d_q, d_out, d_workspace, workspace_bytes, stream);
}

tq_status tq_multi_query_attention_batch(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids,
                                         int32_t n_new, const uint16_t* d_q, float* d_out, void* d_workspace,
                                         size_t workspace_bytes, void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    if ((s = check_seqs(c, layer, n_seq, seq_ids)) != TQ_OK) return s;
    const Dims& dm = c->plan.dm;
    if (n_seq < 1 || n_seq > std::min(MAX_CALL_SEQ, MQ_STREAMS_MAX / dm.hkv))
        return fail(TQ_ERR_INVALID_ARG, "n_seq (%d) must be in [1, %d]", n_seq,
                    std::min(MAX_CALL_SEQ, MQ_STREAMS_MAX / dm.hkv));
    CallSeqs cs{};
    cs.n = n_seq;
    int64_t app[MAX_CALL_SEQ];
    for (int i = 0; i < n_seq; ++i) {
        cs.ids[i] = seq_ids[i];
        app[i] = c->appended[sl_index(dm, seq_ids[i], layer)];
        if (n_new < 1 || n_new > dm.W || n_new > app[i])
            return fail(TQ_ERR_INVALID_ARG,
                        "n_new (%d) must be in [1, min(hot_window %d, tokens appended %lld)] (sequence %d)", n_new,
                        dm.W, (long long)app[i], seq_ids[i]);
    }
    if (!d_q || !d_out || !d_workspace) return fail(TQ_ERR_INVALID_ARG, "a pointer is NULL");
    if ((uintptr_t)d_workspace & 255) return fail(TQ_ERR_INVALID_ARG, "d_workspace must be 256-byte aligned");
    const size_t need = multi_query_workspace_bytes(dm, n_seq);
    if (workspace_bytes < need)
        return fail(TQ_ERR_INVALID_ARG, "workspace of %zu bytes, the call needs %zu", workspace_bytes, need);
    if ((s = flush_pending(c)) != TQ_OK) return s;
    hipError_t e = launch_multi_query(dm, c->P, c->plan.fmts[layer], layer, cs, n_new, app,
                                      reinterpret_cast<const _Float16*>(d_q), d_out,
                                      reinterpret_cast<uint8_t*>(d_workspace), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "multi-query launch");
    return TQ_OK;
}

tq_status tq_get_rotation(tq_cache* c, float* host_pi, float* host_s, void* stream) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    const int d = c->plan.dm.d;
    hipStream_t st = (hipStream_t)stream;
    if (host_pi && (s = sync_copy(host_pi, c->P.pi32, (size_t)d * d * 4, hipMemcpyDeviceToHost, st)) != TQ_OK) return s;
    if (host_s && (s = sync_copy(host_s, c->P.s32, (size_t)M_MAX * d * 4, hipMemcpyDeviceToHost, st)) != TQ_OK) return s;
    return TQ_OK;
}

tq_status tq_profile_enable(tq_cache* c, int32_t enable) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    c->profiling = enable != 0;
    return TQ_OK;
}

tq_status tq_profile_read(tq_cache* c, double* ms_total, int32_t* launches) {
    tq_status s = check_handle(c);
    if (s != TQ_OK) return s;
    double tot = 0.0;
    for (size_t i = 0; i + 1 < c->ev_used; i += 2) {
        hipError_t e = hipEventSynchronize(c->ev_pool[i + 1]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, c->ev_pool[i], c->ev_pool[i + 1]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        tot += ms;
    }
    if (ms_total) *ms_total = tot;
    if (launches) *launches = (int32_t)(c->ev_used / 2);
    c->ev_used = 0;
    return TQ_OK;
}

}  // extern "C"
