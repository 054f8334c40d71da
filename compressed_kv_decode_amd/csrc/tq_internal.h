// Internal layout of a libtqkv arena and the structs passed to kernels.
//
// Everything lives in one caller-owned device arena.  Regions, in order:
//   Pi (fp32 d x d), S (fp32 64 x d), fp16 hi/lo splits of Pi and of S (S's
//   columns permuted to the quantise kernel's MFMA operand order), Pi^T and
//   S^T (fp32, for coalesced per-vector products), S Pi (fp32), error
//   words, per-(seq, layer) metadata, ring tags, tombstone bits, sticky
//   words, promotion candidates, the hot rings (K row-major, V transposed in
//   32-token tiles), the cold code tiles of every layer, and the per-call
//   workspace (rotated queries, split-context partials, append plans).
//
// Cold tiles.  Each (seq, layer, kv_head) owns cold_cap / 32 tile pairs of
// 32 slots; tile pair t is the K tile followed by the V tile, so one decode
// stage is a single contiguous copy.  A tile holds 32 * (PB + SB + 4) bytes,
// PB = (d/2) * code_bits / 8 pair-code bytes and SB = m / 8 sign bytes per
// vector:
//   K tile: [32][PB] token-major records whose pair codes are stored in
//           quarter-major order (position p holds pair perm(p), see
//           pair_of_pos) | [32][SB] sign bits | [32] fp16 R | [32] fp16 rho
//   V tile: [d/2][cb dwords] one row per pair, the code of the token at
//           storage position s at bit s * cb | [m] dwords of sign bits (bit s
//           = storage position s) | [32] fp16 R by token | [32] fp16 rho by
//           storage position
// Value storage position s of token t is vpos(t) (the k order of the value
// accumulation, see vpos); the hot ring's V tiles use the same order.
// K is token-major because a query dots each key's pairs; V is pair-major
// because the output accumulates one pair over many tokens.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq {

constexpr int TILE = 32;        // cold slots per tile
constexpr int M_MAX = 64;       // sketch rows stored (a format uses the first m)
constexpr int MAX_G = 8;        // query heads per kv head
constexpr int MAX_CALL_SEQ = 128;  // sequences per launch batch
// The formats take (radius bits, angle bits) = (2, 3), (3, 4) or (2, 2), so
// the code width CB = rb + tb fixes both.
constexpr int theta_bits_of(int cb) { return cb == 7 ? 4 : (cb == 5 ? 3 : 2); }
constexpr int TC_SEGS = 8;         // segments of a large Tensor Cache write per (sequence, kv head)
constexpr int TC_SEG_MIN = 512;    // tokens of a segment, at least; appends of more new tokens take that path
constexpr int SMALL_APPEND_MAX = 8;  // appends of at most this many tokens per sequence take the fused path
constexpr int ITEMS_MAX = 4096;  // split-context parts per decode launch (each writes two partial records)
constexpr float LO_SCALE = 4096.0f;  // fp16 lo parts are stored times 2^12
constexpr size_t STATIC_WS_BYTES = (size_t)16 << 20;  // workspace of tq_decode_attention_static
constexpr int HOT_SLICES = 4;  // hot-window slices scanned in parallel for the hot-first gate
// device error bits (same values as TQ_DEVERR_* in tqkv.h)
constexpr int DEVERR_R_OVERFLOW = 1;
constexpr int DEVERR_RING_OVERFLOW = 2;
constexpr int DEVERR_COLD_OVERFLOW = 4;

struct SeqLayerMeta {  // one per (seq, layer)
    int32_t head;          // ring index of the oldest hot entry
    int32_t count;         // hot entries
    int32_t cold_len;      // cold slots written
    int32_t attn_step;     // decode-attention calls so far
    int32_t n_promoted;
    int32_t n_evicted;
    int32_t promoted_step; // attn_step seen by the last promote that had candidates
    int32_t done;          // blocks of the running append or promote launch that have finished (0 between launches)
};

struct AppendPlan {  // one per sequence of an append launch
    int32_t nc_old;      // cold_len before the append
    int32_t n_ring_new;  // NEW hot entries evicted (they take the first new slots)
    int32_t e_in;        // input tokens that go straight to cold
    int32_t in_base;     // first input row of this sequence
    int32_t ring_pos;    // ring index of the first input token kept hot
    int32_t n_keep;      // input tokens kept hot
    int32_t nc_new;      // cold_len after the append
    int32_t pad;
};

struct Cand {
    float v;       // logit (per-chunk lists) or probability (final lists)
    int32_t slot;
};

struct CallSeqs {  // sequences of one launch batch, passed by value
    int32_t n;
    int32_t ids[MAX_CALL_SEQ];
    int32_t n_new[MAX_CALL_SEQ];    // append: new tokens; decode: split-context parts per kv head
    int32_t in_base[MAX_CALL_SEQ];  // append: first input row; decode: first split-context item
};

struct Dims {
    int n_seq_max, n_layers, hq, hkv, d, g, W, cap, cold_cap, ktop, max_chunks /* parts per launch */, call_cap;
    float tau;
    int sticky, v_qjl;
    float gate;  // hot-first gate: a kv head's cold slots are skipped when every query head of its
                 // group has a hot logit (natural units) >= gate; +inf: cold always scored
    int tc;      // 1: the Tensor Cache cold tier (evictions write A, no codes)
    float tc_eta, tc_sg;          // write rate, sigmoid of the merge gate
    float tc_log2l;               // log2(tc_lambda) (from fp64)
    float tc_pow[TILE + 1];       // tc_lambda^k, k = 0 .. 32 (from fp64)
    // multi-query attention (0 = a decode step): the queries of the newest
    // mq_n tokens, as virtual heads v = j * mq_g + h (token j, head h of the
    // kv head's group); this launch's head c is virtual head mq_v0 + c
    int mq_n, mq_g, mq_v0;
};

struct Ptrs {
    float* pi32;        // [d][d], y = Pi x
    float* s32;         // [64][d]
    _Float16* pi_hi;    // [d][d] fp16(Pi)
    _Float16* pi_lo;    // [d][d] fp16((Pi - hi) * 2^12)
    _Float16* s_hi;     // [64][d] columns in MFMA operand order
    _Float16* s_lo;
    // the bulk quantiser's copies for a format of tb angle bits, index tb - 2:
    // Pi with each output pair turned by half an angle bin, T Pi, and S T^T
    // (T = the pairwise turn by pi / 2^tb), so that it decides angles on
    // turned pairs directly; same hi/lo splits and orders as pi_hi .. s_lo
    _Float16* tpi_hi;   // [3][d][d]
    _Float16* tpi_lo;
    _Float16* ts_hi;    // [3][64][d]
    _Float16* ts_lo;
    float* pit32;       // [d][d] Pi^T (coalesced columns of Pi)
    float* st32;        // [d][64] S^T
    float* sp32;        // [64][d] S Pi
    int32_t* err;       // [4]
    SeqLayerMeta* meta; // [n_seq_max][n_layers]
    int32_t* tags;      // [n_seq_max][n_layers][cap]: -1 NEW, else source cold slot
    uint32_t* tomb;     // [n_seq_max][n_layers][cold_cap / 32]
    uint32_t* sticky;   // [n_seq_max][n_layers][cold_cap]: (last_step << 8) | count
    Cand* cand;         // [n_seq_max][n_layers][hq][ktop] slots with p >= tau
    int32_t* cand_n;    // [n_seq_max][n_layers][hq]
    _Float16* ring_k;   // [n_seq_max][n_layers][hkv][cap][d]
    _Float16* ring_v;   // [n_seq_max][n_layers][hkv][cap / 32][d][32], tokens at vpos
    uint8_t* cold;      // layer regions, see LayerFmt::off
    uint8_t* tables;    // per-layer decode tables, see LayerFmt::tab_off
    float* qprep;       // [call_cap][hq][d + 64]: Pi q, S Pi q
    float* part;        // [max_chunks parts][hot, cold][g][part_stride] partial records
    Cand* cand_chunk;   // [max_chunks parts][g][ktop] per-part promotion candidates
    _Float16* qgather;  // multi-query passes: the pass's fp16 queries [hkv * g][d] (k_qprep writes, k_decode reads)
    AppendPlan* plan;   // [MAX_CALL_SEQ]
    float* gate_max;    // [call_cap][hkv][HOT_SLICES][MAX_G]: best hot logit per window slice and query head
    float* tc_a;        // [n_seq_max][n_layers][hkv][d][d]: Tensor Cache matrices (tier 1 only)
    float* tc_seg;      // [call_cap][hkv][TC_SEGS][d][d]: segment sums of a large Tensor Cache write
    int32_t* jobs;      // [MAX_CALL_SEQ][cap] ring indices of evicted NEW entries
};

struct LayerFmt {
    int rb, tb, m, cb;   // radius bits, angle bits, sign bits, code bits
    int pb, sb;          // pair-code bytes and sign bytes per vector
    int tile_bytes;      // 32 * (pb + sb + 4)
    size_t off;          // byte offset of the layer's cold region in Ptrs::cold
    float cos_t[16], sin_t[16];  // angle grid -pi + 2 pi b / 2^tb
    float half_c, half_s;        // cos, sin of half an angle bin (pi / 2^tb)
    float cos_h[16], sin_h[16];  // the grid turned by half a bin: -pi + 2 pi (b + 1/2) / 2^tb
    size_t tab_off;              // byte offset of the layer's decode tables in Ptrs::tables
    int pair2;                   // 1: tables indexed by two adjacent codes (code_bits <= 5)
    float vscale, vscale_inv;    // value tables hold fp16(vscale * u); value sums are taken back by vscale_inv
};

// Decode tables of a layer (built on the host at cache creation), in order
// (a decode kernel stages the prefix it uses into LDS):
//   sign table   [16] x 8 B: the four bits of a nibble as fp16 +-1.
//   sign masks   [16] x 8 B: per bit, 0x8000 for a 0 bit (sign -1), else 0.
//   one-code     [2^cb] x 4 B key hi (x, y), then key lo x 2^12 (x, y), then
//                value (x, y), fp16, (x, y) = (a_r / (L_r - 1)) (cos, sin)(phi_b)
//                (value entries times the format's vscale, see value_scale).
//                A table of at most 64 dwords is read without LDS bank
//                conflicts whatever the indices.
//   one-code key pairs [2^cb] x 8 B: fp16 hi (x, y), lo x 2^12 (x, y).
//   two-code value table (code_bits <= 5): [2^(2cb)] x 8 B, fp16 (x of a,
//                x of b, y of a, y of b) for codes a = index & mask,
//                b = index >> cb (one 8-byte read per two tokens), times vscale.
//   two-code key table (code_bits <= 5): [2^(2cb)] x 16 B: fp16 hi (x, y) of
//                a, hi (x, y) of b, lo x 2^12 (x, y) of a, lo (x, y) of b.
// Every block is padded to whole KB.
constexpr int SIGN_TAB_BYTES = 16 * 8;

__host__ __device__ constexpr int onetab_off_of(int) { return 2 * SIGN_TAB_BYTES; }
__host__ __device__ constexpr int khl_off_of(int cb) { return onetab_off_of(cb) + 3 * (4 << cb); }
__host__ __device__ constexpr int v2tab_off_of(int cb) { return khl_off_of(cb) + (8 << cb); }
__host__ __device__ constexpr int k2tab_off_of(int cb) { return v2tab_off_of(cb) + (cb <= 5 ? (8 << (2 * cb)) : 0); }
__host__ __device__ constexpr int tables_end_of(int cb) { return k2tab_off_of(cb) + (cb <= 5 ? (16 << (2 * cb)) : 0); }
__host__ __device__ constexpr int kb_round(int b) { return (b + 1023) / 1024 * 1024; }
__host__ __device__ constexpr int tables_bytes_of(int cb) { return kb_round(tables_end_of(cb)); }

// Storage position of token t (0..31) inside a value tile, and its inverse.
// The value accumulation takes the attention weights straight from the
// logit MFMA's output, whose lane (q, c) holds tokens 16 h + 4 q + r (h, r in
// 0..1, 0..3) as k index 8 q + 4 h + r; storing token t at position vpos(t)
// makes a lane's eight k values eight contiguous positions.
__host__ __device__ constexpr int vpos(int t) { return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3); }
__host__ __device__ constexpr int vtok(int s) { return 16 * ((s & 7) >> 2) + 4 * (s >> 3) + (s & 3); }
__host__ __device__ inline int part_stride(int d) { return 2 + d + M_MAX; }

// Position p of a K record holds pair pair_of_pos(p): quarter q = p / (4 nb)
// of the record holds pairs {16 b + 4 q + j}, nb = d / 32, so that one lane of
// a 16x16x32 MFMA operand finds its pairs contiguous.
__host__ __device__ constexpr int pair_of_pos(int p, int d) {
    return 16 * ((p % (d / 8)) / 4) + 4 * (p / (d / 8)) + (p % 4);
}

__host__ __device__ inline size_t sl_index(const Dims& dm, int seq, int layer) {
    return (size_t)seq * dm.n_layers + layer;
}

__host__ __device__ inline size_t cold_tile_offset(const Dims& dm, const LayerFmt& f, int seq, int kvh,
                                                   int kv, int tile) {
    size_t ntile = (size_t)dm.cold_cap / TILE;
    return f.off + ((((size_t)seq * dm.hkv + kvh) * ntile + tile) * 2 + kv) * (size_t)f.tile_bytes;
}

__host__ __device__ inline size_t ring_base(const Dims& dm, int seq, int layer, int kvh) {
    return ((sl_index(dm, seq, layer) * dm.hkv) + kvh) * (size_t)dm.cap * dm.d;
}

// Launchers (defined next to their kernels).
// Fp, layer_p >= 0 and fused != NULL: a small append also runs the
// promotion of layer layer_p (format Fp, the same code width as F) of the
// same sequences in its launch and sets *fused (else the caller launches that
// promotion itself).  q != NULL and q_done != NULL: a small append also
// prepares the queries q of this layer's ungated attention step (sketch
// scale cm) in its launch and sets *q_done (else the attention launch does).
hipError_t launch_append(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs,
                         int max_new, const _Float16* k, const _Float16* v, hipStream_t st,
                         const LayerFmt* Fp = nullptr, int layer_p = -1, bool* fused = nullptr,
                         const _Float16* q = nullptr, float cm = 0.0f, bool* q_done = nullptr);
// Scale of the sketch part of the prepared query, sqrt(pi/2) / m.
float qjl_query_scale(const LayerFmt& F);
hipError_t launch_evict(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs, int target_hot,
                        hipStream_t st);
hipError_t launch_decode(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, CallSeqs cs,
                         const int64_t* appended, const _Float16* q, float* out, float* logits, int logits_stride,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, bool q_ready = false);
// Tensor Cache writes of the tokens an append plan evicts (k, v: the
// append's input rows; max_new: the most new tokens of a sequence, which
// selects the segmented MFMA path for large appends).
hipError_t launch_tc_write(const Dims& dm, const Ptrs& P, int layer, const CallSeqs& cs, int max_new,
                           const _Float16* k, const _Float16* v, hipStream_t st);
// Compressed-vector search over the cold slots of (seq, layer, kv head):
// the k best code-domain inner products per query.  ws: the workspace
// (mips_workspace_bytes; appended: the stream's appended tokens).
size_t mips_workspace_bytes(const Dims& dm, int n_q, int k, int64_t appended);
hipError_t launch_mips(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, int seq, int kvh, int n_q,
                       const _Float16* q, int k, int32_t* idx, float* score, uint8_t* ws, int64_t appended,
                       hipStream_t st);
// The search scan (k_mips_scan) over n_groups groups of 8 prepared queries,
// n_parts parts of the stream: each (group, part) writes its best k per query.
hipError_t launch_mips_scan(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, int seq, int kvh,
                            int n_groups, int n_parts, int k, Cand* part, hipStream_t st);
// Multi-query attention of the newest n_new tokens of each sequence of seqs
// (appended: their token counts; ws: the caller's workspace of
// multi_query_workspace_bytes for seqs.n sequences).
constexpr int MQ_STREAMS_MAX = 2048;  // (sequence, kv head) streams per call: one part each at least
size_t multi_query_workspace_bytes(const Dims& dm, int n_seq);
hipError_t launch_multi_query(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& seqs,
                              int n_new, const int64_t* appended, const _Float16* q, float* out, uint8_t* ws,
                              hipStream_t st);
// k_qprep over n_groups groups of 8 queries q [n_groups * 8][d] into P.qprep.
hipError_t launch_qprep8(const Dims& dm, const Ptrs& P, const _Float16* q, int n_groups, float cm, hipStream_t st);
hipError_t launch_promote(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs,
                          hipStream_t st);
hipError_t launch_clear(void* p, size_t bytes, hipStream_t st);
// This GPU's copy of the static decode workspace (STATIC_WS_BYTES; its device
// address, looked up once per device).
hipError_t static_workspace(void** ptr);
// Read-only bandwidth probe over bytes (a multiple of 16) of buf; sink holds
// one word per block.
hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t st);

}  // namespace tq
