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
 *    sketch.  Here: y = Pi x with a seeded rotation Pi (Haar, or randomized
 *    Hadamard: tq_config.rotation_kind); per adjacent
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

#define TQKV_VERSION 0x00010500u /* 1.5.0 */

/* Rotations (tq_config.rotation_kind), used when tq_config.rotation is NULL. */
#define TQ_ROTATION_HAAR 0     /* dense Haar: Q of the QR of a seeded Gaussian matrix (default) */
#define TQ_ROTATION_HADAMARD 1 /* randomized Hadamard: Walsh matrix times seeded column signs / sqrt(d) */

/* Cold tiers (tq_config.cold_tier). */
#define TQ_COLD_CODES 0        /* evicted tokens become packed codes (default) */
#define TQ_COLD_TENSOR_CACHE 1 /* evicted tokens are written into a d x d outer-product matrix */

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
    /* Cold tier.  TQ_COLD_TENSOR_CACHE follows "Tensor Cache:
     * Eviction-conditioned Associative Memory for Transformers"
     * (gist.science), section "Metodologia": each (sequence, layer, kv head)
     * holds A (d x d, fp32, zero at creation); every token the window evicts
     * is written A <- tc_lambda A + tc_eta (k outer v), oldest first, and is
     * not kept otherwise; decode attention is exact softmax over the hot
     * window plus sigmoid(tc_gate) q A.  The page learns these scalars; here
     * they are fixed.  Requires promote_threshold > 1 (no individual cold
     * tokens to promote). */
    int32_t cold_tier;     /* TQ_COLD_CODES or TQ_COLD_TENSOR_CACHE          */
    float tc_lambda;       /* decay, in (0, 1]                               */
    float tc_eta;          /* write rate, finite                             */
    float tc_gate;         /* g of the merge (sigmoid(g) scales the read)    */
    /* The rotation drawn from the seed when rotation is NULL.  "TurboQuant:
     * kompresja KV-cache w LLM 6 razy" (sudonull.com), section "Zasada
     * dzialania PolarQuant", names a random rotation without its kind: a
     * dense Haar matrix by default, or a randomized Hadamard matrix
     * (Pi[i][j] = (-1)^popcount(i & j) s_j / sqrt(d), s_j = -1 where the top
     * bit of output j of SplitMix64 stream 2 of the seed is set).  Both are
     * applied as dense matrices on the MFMA units. */
    int32_t rotation_kind; /* TQ_ROTATION_HAAR or TQ_ROTATION_HADAMARD        */
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
 * bytes, 256-byte aligned).
 * Defined by: "TurboQuant: kompresja KV-cache w LLM 6 razy bez utraty
 * dokladnosci" (sudonull.com), section "Zasada dzialania PolarQuant" (the
 * vector is first rotated at random: the seeded rotation Pi made here)
 * and section "Kompensacja bledow przez QJL" (the Johnson-Lindenstrauss
 * projection whose signs code the residual: the Gaussian sketch S); "Monarch
 * v3" (openclawradar.com), section "Como funciona" (a hot region of recent
 * full-precision tokens and a compressed cold region: the arena's ring and
 * cold slots).  The arena must outlive the handle.  ASYNC: the
 * rotation Pi and sketch S (generated on the host in fp64 from the seed --
 * SplitMix64 streams, Box-Muller normals, Householder QR with R's diagonal
 * made positive for the Haar rotation, the Walsh matrix times seeded column
 * signs for the randomized Hadamard one -- or taken from cfg) are copied to
 * the arena and all
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
 * Defined by: "Monarch v3" (openclawradar.com), section "Como funciona"
 * (sliding window: the newest tokens stay hot, older ones are compressed to
 * the cold region) and section "Bucle de Decodificacion Simplificado" (when
 * the hot window overflows the oldest entry goes to cold); the quantisation
 * of an evicted entry follows "TurboQuant: kompresja KV-cache w LLM 6 razy"
 * (sudonull.com), sections "Zasada dzialania PolarQuant" (rotate, radius and
 * angle, quantise) and "Kompensacja bledow przez QJL" (1-bit sketch of the
 * residual), and steps two to five of the quantisation flow of "TurboQuant:
 * optimizacion de memoria para KV caches" (kerneldigest.dev).
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
 * Defined by: "TurboQuant: optimizacion de memoria para KV caches en
 * inferencia de LLMs" (kerneldigest.dev), step six of the quantisation flow
 * (attention logits computed from the compressed cache) and section
 * "Arquitectura del Sistema" (the QJL correction keeps the scores accurate);
 * "TurboQuant: kompresja KV-cache w LLM 6 razy" (sudonull.com), section
 * "Kompensacja bledow przez QJL" (the sign code's inner-product estimate);
 * "Monarch v3" (openclawradar.com), section "Bucle de Decodificacion
 * Simplificado" (the hot window is scored at full precision beside the cold
 * pages).
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

/* One decode step of one layer in one call: tq_quantize_append(c, layer,
 * n_seq, seq_ids, n_new, d_k, d_v, stream), then tq_decode_attention(c,
 * layer, n_seq, seq_ids, d_q, d_out, NULL, stream); the results, the
 * recorded promotion candidates and the cache state are exactly theirs.
 * Defined by: "Monarch v3" (openclawradar.com), section "Bucle de
 * Decodificacion Simplificado" (a decode step appends the new token, evicting
 * the oldest hot entry to cold when the window overflows, and attends over
 * hot and cold), with the passages cited at those two calls.  When the
 * appends are small (at most 8 tokens per sequence, the decode-step case)
 * and the attention runs as one batch (n_seq <= 128 and n_seq * n_kv_heads
 * <= 4096), the queries are taken into the rotated domain inside the append's
 * launch (which may also run a promotion deferred by tq_promote_deferred),
 * so the step takes one launch fewer.  Arguments as in the two calls.  All
 * arguments are checked before anything is launched.  ASYNC.  Errors: as
 * tq_quantize_append and tq_decode_attention. */
tq_status tq_decode_step(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, const int32_t* n_new,
                         const uint16_t* d_k, const uint16_t* d_v, const uint16_t* d_q, float* d_out,
                         void* stream);

/* tq_decode_attention with the hot-first gate of "Monarch v3"
 * (openclawradar.com), section "Bucle de Decodificacion Simplificado": the
 * cold pages are scored only when the best hot score falls below a
 * threshold, since the recent window usually holds the attention (section
 * "Limitaciones" names this recency assumption).  Per (sequence, kv head):
 * the hot logits <q, k>/sqrt(head_dim) of every query head of the group are
 * computed first; if each head's best one is >= threshold the group's cold
 * slots are not read and its heads attend over the hot entries only (their
 * debug logits stay -inf on the cold side and they record no promotion
 * candidates); otherwise the step is tq_decode_attention's.  An empty hot
 * window never gates.  threshold = +inf is tq_decode_attention.  ASYNC.
 * Errors: as tq_decode_attention, plus TQ_ERR_INVALID_ARG for a NaN
 * threshold. */
tq_status tq_decode_attention_gated(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids,
                                    const uint16_t* d_q, float* d_out, float* d_logits_dbg, float threshold,
                                    void* stream);

/* tq_decode_attention for callers that cannot allocate or reserve device
 * memory per call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and recorded
 * promotion candidates as tq_decode_attention; the call's scratch (rotated
 * queries, split-context partial records, per-part candidates) lives in a
 * static device array of the library instead of the arena's workspace:
 * 16 MiB, one copy per GPU the library runs on, held until the process ends.
 * Batches of sequences are cut so that each fits; a configuration whose
 * single sequence does not fit (n_q_heads * (head_dim + 64) * 4 bytes of
 * queries plus n_kv_heads * (2 * group * (head_dim + 66) * 4 + group *
 * max(1, floor(1/tau)) * 8) bytes per part) is rejected with
 * TQ_ERR_CAPACITY.  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads, other caches) race and
 * must be ordered by the caller.  Allocates nothing (no hipMalloc, no
 * events).  ASYNC.  Errors: TQ_ERR_INVALID_ARG, TQ_ERR_CAPACITY,
 * TQ_ERR_HIP. */
tq_status tq_decode_attention_static(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids,
                                     const uint16_t* d_q, float* d_out, float* d_logits_dbg, void* stream);

/* Promotion after the last tq_decode_attention of this layer for these
 * sequences.  Defined by: "Monarch v3" (openclawradar.com), section "Como
 * funciona" (attention-weighted promotion of cold tokens with a sticky
 * mechanism against thrashing), section "Bucle de Decodificacion
 * Simplificado" (cold pages with high attention move to hot for the next
 * step) and section "Como probarlo" (the promotion threshold and sticky
 * count as parameters).  Semantics: per cold slot c, P_c = max over the layer's query heads of its
 * probability; the sticky counter of c counts consecutive steps with
 * P_c >= tau (reset otherwise); slots whose counter reaches ``sticky`` are
 * dequantised (QJL term included) to fp16 and enter the hot window as the
 * newest entries (P_c descending, ties to the lower slot), and their cold
 * slot is tombstoned.  No-op when tau > 1.  ASYNC.  Errors:
 * TQ_ERR_INVALID_ARG, TQ_ERR_STATE (no attention on a sequence since its
 * last promote), TQ_ERR_HIP. */
tq_status tq_promote(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, void* stream);

/* tq_promote whose launch may be deferred, for decode loops that run one
 * stream: the promotion is kept in the handle and launched by the next call
 * on it.  When that call is tq_quantize_append of another layer of exactly
 * these sequences (same order) on the same stream, with a small append (a
 * decode step) and the same code and sketch widths, the promotion runs inside
 * the append's launch (the two touch disjoint state); every other call
 * launches it first, on the stream it was issued on.  tq_cache_destroy drops
 * it.  The result is the same as tq_promote's.  Work the caller orders after
 * this call by other means (an event recorded on the stream, another stream)
 * must be preceded by tq_flush.  Defined by the same passages as tq_promote.
 * ASYNC.  Errors: as tq_promote (a deferred launch's TQ_ERR_HIP is reported
 * by the call that launches it). */
tq_status tq_promote_deferred(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids, void* stream);

/* Launches a promotion deferred by tq_promote_deferred now, on the stream it
 * was issued on; nothing when none is pending.  ASYNC.  Errors:
 * TQ_ERR_INVALID_ARG, TQ_ERR_HIP. */
tq_status tq_flush(tq_cache* c);

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

/* Multi-query attention over the compressed cache: the queries of the newest
 * n_new tokens of one sequence -- a prefill chunk, or draft tokens being
 * verified -- after tq_quantize_append has appended them (still hot:
 * n_new <= hot_window).  Query j (0 = the oldest of the chunk) attends over
 * every live cold slot and the hot entries up to its own token; cold logits
 * and values are read from the codes as in tq_decode_attention ("TurboQuant:
 * optimizacion de memoria para KV caches" (kerneldigest.dev), step six of
 * the quantisation flow; "Compresion del cache KV de los LLM a 3 bits"
 * (sudonull.com), the long-context processing the codec speeds up).  The
 * call records no promotion candidates and does not count as a decode step.
 *   d_q: device fp16 [n_new, n_q_heads, head_dim]; d_out: device fp32, same
 *   shape.  d_workspace: device, 256-byte aligned, >=
 *   tq_multi_query_workspace_bytes.
 * ASYNC.  Errors: TQ_ERR_INVALID_ARG, TQ_ERR_HIP. */
tq_status tq_multi_query_workspace_bytes(const tq_cache* c, size_t* bytes);
tq_status tq_multi_query_attention(tq_cache* c, int32_t layer, int32_t seq, int32_t n_new, const uint16_t* d_q,
                                   float* d_out, void* d_workspace, size_t workspace_bytes, void* stream);

/* tq_multi_query_attention for a batch of sequences in one call (a batched
 * prefill chunk, or the draft tokens of every sequence of a speculative
 * decoding batch): each sequence's newest n_new tokens (the same n_new for
 * all), with the semantics above per sequence.  The sequences share each
 * pass's launches, so the cold tiles of the whole batch stream through one
 * split-context launch per pass.  Defined by the same passages.
 *   seq_ids: host [n_seq], distinct; 1 <= n_seq <= min(128, 2048 / n_kv_heads).
 *   d_q: device fp16 [n_seq, n_new, n_q_heads, head_dim], sequences in
 *   seq_ids order; d_out: device fp32, same shape.  d_workspace: device,
 *   256-byte aligned, >= tq_multi_query_batch_workspace_bytes(c, n_seq).
 * ASYNC.  Errors: TQ_ERR_INVALID_ARG, TQ_ERR_HIP. */
tq_status tq_multi_query_batch_workspace_bytes(const tq_cache* c, int32_t n_seq, size_t* bytes);
tq_status tq_multi_query_attention_batch(tq_cache* c, int32_t layer, int32_t n_seq, const int32_t* seq_ids,
                                         int32_t n_new, const uint16_t* d_q, float* d_out, void* d_workspace,
                                         size_t workspace_bytes, void* stream);

/* Compressed-vector maximum inner-product search over the cold slots of one
 * (seq, layer, kv_head) stream ("Compresion del cache KV de los LLM a 3
 * bits: TurboQuant" (sudonull.com), section "Aplicaciones mas alla de los
 * LLMs": the codec stored vectors are searched by estimated inner products).
 * Vectors enter the store through tq_quantize_append (as keys) followed by
 * tq_evict to 0, which leaves every one in a cold slot, slot j = the j-th
 * appended.  The score of slot j for query q is the code-domain estimate
 * <Pi q, y_hat_j> + sqrt(pi/2)/m rho_j <S_m Pi q, sigma_j> (the decode
 * path's cold logit times sqrt(head_dim)); tombstoned slots and hot entries
 * are not searched.
 *   d_q: device fp16 [n_q, head_dim], 1 <= n_q <= TQ_MIPS_MAX_QUERIES.
 *   d_idx, d_score: device int32 / fp32 [n_q, k], 1 <= k <= TQ_MIPS_MAX_K:
 *        the k best slots per query, score descending, the lower slot first
 *        on equal scores; -1 / -inf where fewer than k slots exist.
 *   d_workspace: device, 256-byte aligned, >= tq_mips_workspace_bytes.
 * ASYNC.  Errors: TQ_ERR_INVALID_ARG, TQ_ERR_STATE (a tensor-cache tier
 * cache), TQ_ERR_HIP. */
#define TQ_MIPS_MAX_K 32
#define TQ_MIPS_MAX_QUERIES 4096
tq_status tq_mips_workspace_bytes(const tq_cache* c, int32_t n_q, int32_t k, size_t* bytes);
tq_status tq_mips_search(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, int32_t n_q, const uint16_t* d_q,
                         int32_t k, int32_t* d_idx, float* d_score, void* d_workspace, size_t workspace_bytes,
                         void* stream);

/* BLOCKING test aid (TQ_COLD_TENSOR_CACHE caches): the matrix A of (seq,
 * layer, kv_head), fp32 [head_dim][head_dim] row-major (A[i][j] accumulates
 * k_i v_j), into host_a.  TQ_ERR_STATE for a cache with the codes tier. */
tq_status tq_export_tensor_cache(tq_cache* c, int32_t seq, int32_t layer, int32_t kv_head, float* host_a,
                                 void* stream);

/* BLOCKING.  The fp32 rotation [d*d] and sketch [64*d] in use (either may
 * be NULL). */
tq_status tq_get_rotation(tq_cache* c, float* host_pi, float* host_s, void* stream);

/* Hot-window slots (hot_window plus promotion headroom, rounded to 32) and
 * the per-sequence debug-logit stride of tq_decode_attention. */
tq_status tq_cache_geometry(const tq_cache* c, int32_t* hot_capacity, int32_t* logits_stride);

/* Measurement aid: one read-only pass over bytes (a positive multiple of
 * 16; d_buf 16-byte aligned) of device memory d_buf, 16-byte loads spread
 * over ``blocks`` blocks of 512 threads, each block writing one XOR word to
 * d_sink [blocks] (device).  Timed by the caller (events around the call), it
 * gives the HBM bandwidth a kernel that only reads reaches, the ceiling of a
 * scan over the compressed cache.  ASYNC.  Errors: TQ_ERR_INVALID_ARG,
 * TQ_ERR_HIP. */
tq_status tq_probe_read_bandwidth(const void* d_buf, size_t bytes, uint32_t* d_sink, int32_t blocks, void* stream);

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
