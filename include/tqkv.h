/*
 * libtqkv -- decode attention over a compressed KV cache on AMD Instinct
 * MI355X (gfx950).  C ABI.
 *
 * What the library computes (pages cited by title and section):
 *
 *  - Codec.  "TurboQuant: kompresja KV-cache w LLM 6 razy bez utraty
 *    dokladnosci" (sudonull.com), section "Zasada dzialania PolarQuant": a
 *    vector is rotated at random, then described by radius and angle, which
 *    are quantised; section "Kompensacja bledow przez QJL": the quantisation
 *    residual is coded with one bit per projection of a Johnson-Lindenstrauss
 *    sketch.  Here: y = Pi x with a seeded Haar rotation Pi; per adjacent
 *    coordinate pair (y[2i], y[2i+1]) a radius code (r_bits, uniform on
 *    [0, R], R = fp16 of the largest pair radius) and an angle code
 *    (theta_bits, uniform on [-pi, pi)); the residual's norm (fp16) and the
 *    signs of S_m (y - y_hat) for an m x d Gaussian sketch S_m.
 *  - Attention on codes.  "TurboQuant: optimizacion de memoria para KV
 *    caches en inferencia de LLMs" (kerneldigest.dev), seven-step flow, step
 *    six: logits are computed from the compressed cache.  A cold logit is
 *    [<Pi q, y_hat> + sqrt(pi/2)/m * rho * <S_m Pi q, sign(S_m e)>] / sqrt(d);
 *    cold values are dequantised on the fly.
 *  - Paging.  "Monarch v3: Paginacion KV Inspirada en NES"
 *    (openclawradar.com), section "Como funciona": a hot window of recent
 *    tokens at fp16, older tokens compressed to cold slots by sliding-window
 *    eviction, attention-weighted promotion back to hot with a sticky
 *    counter; section "Bucle de Decodificacion Simplificado": attend,
 *    promote for the next step, evict the oldest when the window overflows.
 *
 * Conventions for every call:
 *  - Every call returns tq_status (TQ_OK == 0).  No C++ exception crosses
 *    the ABI.  On failure tq_last_error() describes the cause (thread-local).
 *  - Arguments are validated on the host before anything is launched; an
 *    invalid call changes no state.
 *  - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls marked ASYNC only enqueue work on that stream and never
 *    synchronise; their device pointers must stay valid until the stream
 *    reaches them.  Calls marked BLOCKING synchronise the stream.
 *  - Device pointers are HIP device memory on the current device; host
 *    pointers are ordinary host memory.  fp16 values are passed as uint16_t
 *    bit patterns (IEEE binary16).
 *  - The library never allocates device memory: the caller owns the arena
 *    and all inputs and outputs.  The handle is library-owned host memory.
 *  - One host thread at a time per handle; calls on one handle must be
 *    ordered by the caller (one stream, or events between streams).
 *  - Errors found by kernels (an fp16 overflow of a radius scale, a ring or
 *    cold overflow that host checks could not see) are latched in the arena
 *    and reported by tq_cache_sync_stats().
 */
#ifndef TQKV_H
#define TQKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQKV_VERSION 0x00010000u /* 1.0.0 */

typedef enum tq_status {
    TQ_OK = 0,
    TQ_ERR_INVALID_ARG = 1, /* null pointer, out-of-range index or size    */
    TQ_ERR_UNSUPPORTED = 2, /* head_dim, bit widths or m not built         */
    TQ_ERR_CAPACITY = 3,    /* an append would exceed max_context          */
    TQ_ERR_STATE = 4,       /* call order violated (e.g. promote twice)    */
    TQ_ERR_HIP = 5,         /* a HIP runtime call failed                   */
    TQ_ERR_DEVICE = 6,      /* a kernel latched an error (see sync_stats)  */
    TQ_ERR_HOST_ALLOC = 7   /* host memory for the handle could not be had */
} tq_status;

/* Code format of one layer.  Built combinations: (r_bits, theta_bits) in
 * {(2,3), (3,4), (2,2)} with qjl_m in {32, 64}; F3 = (2,3,32),
 * F4 = (3,4,64), F2.5 = (2,2,64). */
typedef struct tq_format {
    uint8_t r_bits;     /* radius code bits per pair (levels 2^r_bits)    */
    uint8_t theta_bits; /* angle code bits per pair (angles 2^theta_bits) */
    uint16_t qjl_m;     /* QJL sign bits per vector                      */
} tq_format;

typedef struct tq_config {
    int32_t n_seq_max;   /* sequences the cache holds (ids 0..n_seq_max-1) */
    int32_t n_layers;
    int32_t n_q_heads;   /* multiple of n_kv_heads; group size <= 8        */
    int32_t n_kv_heads;
    int32_t head_dim;    /* 64 or 128                                      */
    int32_t hot_window;  /* W: hot entries kept after each append, >= 1    */
    int32_t max_context; /* tokens one sequence may ever append            */
    const tq_format* layer_formats; /* host array [n_layers], copied      */
    uint64_t seed;       /* seeds the rotation and the sketch              */
    float promote_threshold; /* tau; > 1 disables promotion; else >= 1/64  */
    int32_t sticky;      /* consecutive qualifying steps to promote, >= 1  */
    int32_t v_qjl;       /* 1: dequantised values include the QJL term     */
    const float* rotation; /* optional host [d*d] row-major Pi (y = Pi x); NULL: from seed */
    const float* sketch;   /* optional host [64*d] row-major S; NULL: from seed */
} tq_config;

typedef struct tq_cache tq_cache;

typedef struct tq_stats {
    int32_t hot_len;        /* entries in the hot window                   */
    int32_t cold_len;       /* cold slots written (append-only)            */
    int32_t live_cold;      /* cold slots not tombstoned                   */
    int32_t n_promoted;     /* promotions so far                           */
    int32_t n_evicted;      /* evictions so far (NEW and PROMOTED)         */
    int32_t attn_steps;     /* decode-attention calls on this (seq, layer) */
    int32_t device_error;   /* latched kernel error bits (0 = none)        */
    int32_t hot_capacity;   /* ring slots (W plus promotion headroom)      */
    int64_t tokens_appended;
} tq_stats;

/* Device error bits reported in tq_stats.device_error. */
#define TQ_DEVERR_R_OVERFLOW 1    /* a pair radius exceeded the fp16 range  */
#define TQ_DEVERR_RING_OVERFLOW 2 /* promotions exceeded the ring headroom  */
#define TQ_DEVERR_COLD_OVERFLOW 4 /* cold slots exceeded the capacity       */

/* Arena bytes a configuration needs.  Pure host, touches no device.
 * Errors: TQ_ERR_INVALID_ARG (null pointer, non-positive sizes, tau/sticky
 * out of range), TQ_ERR_UNSUPPORTED (head_dim, formats or group size not
 * built). */
tq_status tq_cache_required_bytes(const tq_config* cfg, size_t* arena_bytes);

/* Create a cache over caller-owned device memory d_arena (>= the required
 * bytes, 256-byte aligned).  The arena must outlive the handle.  ASYNC: the
 * rotation Pi and sketch S (generated on the host in fp64 from the seed --
 * SplitMix64 streams, Box-Muller normals, Householder QR with R's diagonal
 * made positive -- or taken from cfg) are copied to the arena and all
 * metadata is cleared on ``stream``.  *out receives the handle.  Errors: as
 * tq_cache_required_bytes, plus TQ_ERR_INVALID_ARG for a short or unaligned
 * arena, TQ_ERR_HIP, TQ_ERR_HOST_ALLOC. */
tq_status tq_cache_create(const tq_config* cfg, void* d_arena, size_t arena_bytes, void* stream,
                          tq_cache** out);

/* Free the handle (never the arena).  TQ_ERR_INVALID_ARG on a null or
 * already destroyed handle. */
tq_status tq_cache_destroy(tq_cache* c);

/* Append tokens to the hot window of one layer for n_seq sequences, then
 * evict the oldest hot entries (FIFO) until at most hot_window remain: an
 * evicted NEW entry is quantised into the next cold slot (rotation,
 * pair codes, residual sketch, packed store); an evicted PROMOTED entry
 * revives its tombstoned cold slot.  Prefill and decode use the same call.
 *   seq_ids: host [n_seq], distinct, each < n_seq_max.
 *   n_new:   host [n_seq], tokens per sequence (>= 0).
 *   d_k, d_v: device fp16 [sum(n_new), n_kv_heads, head_dim], sequences in
 *            seq_ids order, tokens oldest first.  May be NULL if
 *            sum(n_new) == 0.
 * ASYNC.  Errors: TQ_ERR_INVALID_ARG, TQ_ERR_CAPACITY (host mirror predicts
 * more than max_context tokens for a sequence), TQ_ERR_HIP. */
tq_status tq_quantize_append(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids,
                             const int32_t* n_new, const uint16_t* d_k, const uint16_t* d_v,
                             void* stream);

/* One decode-attention step of one layer: softmax attention of d_q over
 * every live token (hot entries read as fp16, cold slots read from their
 * codes), split over the context and merged.
 *   d_q:   device fp16 [n_seq, n_q_heads, head_dim] (query head h reads kv
 *          head h / (n_q_heads / n_kv_heads)).
 *   d_out: device fp32 [n_seq, n_q_heads, head_dim].
 *   d_logits_dbg: NULL, or device fp32 [n_seq, n_q_heads, hot_capacity +
 *          round_up(max_context, 32)]: entries [0, hot_capacity) are the
 *          hot entries in FIFO order (oldest first), then cold slot j at
 *          hot_capacity + j; -inf where no live token is.  Logits include
 *          the 1/sqrt(head_dim) scale.
 * Records, per (sequence, layer), the cold slots whose probability reaches
 * the promotion threshold, for tq_promote.  ASYNC.  Errors:
 * TQ_ERR_INVALID_ARG, TQ_ERR_HIP. */
tq_status tq_decode_attention(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids,
                              const uint16_t* d_q, float* d_out, float* d_logits_dbg, void* stream);

/* Promotion after the last tq_decode_attention of this layer for these
 * sequences: per cold slot c, P_c = max over the layer's query heads of its
 * probability; the sticky counter of c counts consecutive steps with
 * P_c >= tau (reset otherwise); slots whose counter reaches ``sticky`` are
 * dequantised (QJL term included) to fp16 and enter the hot window as the
 * newest entries (P_c descending, ties to the lower slot), and their cold
 * slot is tombstoned.  No-op when tau > 1.  ASYNC.  Errors:
 * TQ_ERR_INVALID_ARG, TQ_ERR_STATE (no attention on a sequence since its
 * last promote), TQ_ERR_HIP. */
tq_status tq_promote(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, void* stream);

/* Eviction without an append (a test aid): while more than target_hot
 * entries are hot, the oldest is evicted exactly as tq_quantize_append
 * evicts ("Monarch v3", sections "Como funciona" and "Bucle de
 * Decodificacion Simplificado": the oldest hot tokens go to the compressed
 * region) -- a NEW entry is quantised into the next cold slot, a PROMOTED
 * entry revives its tombstoned slot.
 *   target_hot: >= 0; a sequence with at most target_hot hot entries is
 *               left as it is.
 * ASYNC.  Errors: TQ_ERR_INVALID_ARG, TQ_ERR_HIP. */
tq_status tq_evict(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, int32_t target_hot,
                   void* stream);

/* BLOCKING.  Counters of one (sequence, layer) and the latched device error
 * bits.  Returns TQ_ERR_DEVICE when an error bit is set (out is filled). */
tq_status tq_cache_sync_stats(tq_cache* c, int32_t seq, int32_t layer, tq_stats* out, void* stream);

/* BLOCKING test and checkpoint aid.  Canonical records of cold slots
 * [first_slot, first_slot + n) of (seq, layer, kv_head, kv: 0 = K, 1 = V),
 * whatever the internal tiling: per record ceil(P*(r_bits+theta_bits)/8)
 * bytes of pair codes c_i = a_i | (b_i << r_bits) at bit i*(r_bits +
 * theta_bits) (least significant bit first), then qjl_m/8 bytes of sign
 * bits, then R and rho as little-endian fp16.  host_out: n * record bytes. */
tq_status tq_export_codes(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, int32_t kv,
                          int32_t first_slot, int32_t n, uint8_t* host_out, void* stream);

/* BLOCKING test and checkpoint aid, inverse of tq_export_codes: write
 * canonical records into cold slots [first_slot, first_slot + n), which must
 * lie below the slots already written (it overwrites codes, it does not
 * append). */
tq_status tq_import_codes(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, int32_t kv,
                          int32_t first_slot, int32_t n, const uint8_t* host_in, void* stream);

/* BLOCKING test aid.  The hot window of (seq, layer) in FIFO order:
 *   *n_hot receives the entry count; host_tags [hot_capacity] receives -1
 *   for a NEW entry or the cold slot a PROMOTED entry came from;
 *   host_k, host_v (each may be NULL): fp16 [n_kv_heads, hot_capacity,
 *   head_dim], entries in FIFO order. */
tq_status tq_export_hot(tq_cache* c, int32_t seq, int32_t layer, int32_t* n_hot, int32_t* host_tags,
                        uint16_t* host_k, uint16_t* host_v, void* stream);

/* BLOCKING test aid.  For cold slots [0, n) of (seq, layer): host_live[j] =
 * 1 unless tombstoned; host_sticky[j] = the consecutive qualifying steps
 * counted up to the last attention step (0 if it missed that step). */
tq_status tq_export_paging(tq_cache* c, int32_t seq, int32_t layer, int32_t n, uint8_t* host_live,
                           int32_t* host_sticky, void* stream);

/* BLOCKING.  The fp32 rotation [d*d] and sketch [64*d] in use (either may
 * be NULL). */
tq_status tq_get_rotation(tq_cache* c, float* host_pi, float* host_s, void* stream);

/* Hot-window slots (hot_window plus promotion headroom, rounded to 32) and
 * the per-sequence debug-logit stride of tq_decode_attention. */
tq_status tq_cache_geometry(const tq_cache* c, int32_t* hot_capacity, int32_t* logits_stride);

/* Kernel timing for measurement tools.  While enabled, tq_decode_attention
 * records a pair of HIP events around its split-context attention kernel
 * (the dominant kernel) on the caller's stream.  tq_profile_read
 * synchronises, returns the summed milliseconds and launch count since the
 * last read, and clears them. */
tq_status tq_profile_enable(tq_cache* c, int32_t enable);
tq_status tq_profile_read(tq_cache* c, double* ms_total, int32_t* launches);

const char* tq_status_string(tq_status s);
const char* tq_last_error(void);
uint32_t tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQKV_H */
