/*
 * tq.h — C ABI of the TurboQuant compressed-KV library for AMD MI355X (gfx950).
 *
 * What the library computes (sources cited by page title and section):
 *
 *  - Encoding of attention keys with the product quantizer TurboQuantProd: a
 *    fixed random orthogonal rotation Pi of the unit key, one Lloyd-Max scalar
 *    quantizer shared by every rotated coordinate, and a 1-bit QJL sign sketch
 *    sign(S r) of the residual r together with |r|  (page "TurboQuant — Random
 *    rotation trước khi quantize, 3-bit KV cache không mất accuracy",
 *    section "Ý tưởng cốt lõi"; page "turboquant/audit_claims.py", AUDIT 3 and
 *    AUDIT 5 for the TurboQuantProd(bits) interface).
 *  - Encoding of values either with the asymmetric min/max group code of the
 *    compressed store (page "turboquant/audit_claims.py", AUDIT 1:
 *    value_bits, value_group_size) or with the same rotated Lloyd-Max code.
 *  - Single-query decode attention that reads only the compressed cache plus a
 *    bf16 ring of recent tokens: scores from the rotated query against the
 *    codebook-indexed keys plus the QJL correction, online softmax, values
 *    decoded on chip (page "03. Results & Benchmarks", sections "Latency
 *    Benchmarks" and "Next Steps"; rotate the query at run time: page
 *    "TurboQuant — ...", section "Tại sao nó hoạt động").
 *    Variants: several causal queries per sequence (AUDIT 4's T axis) and a
 *    decode step with the ring append fused in.
 *  - Byte accounting of the cache (page "turboquant/audit_claims.py", AUDIT 1).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the argument name ends in _host.
 *    Every buffer is owned by the caller; the library never allocates or
 *    frees device memory.  It keeps no state between calls, apart from the
 *    static device scratch of tq_decode_attn_noalloc.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Device work is
 *    enqueued on it asynchronously; a device fault surfaces at the caller's
 *    next synchronisation.
 *  - Return value: TQ_OK (0) or a negative TQ_ERR_* code.  Every argument is
 *    checked on the host before anything is launched, so a call that returns
 *    an error other than TQ_ERR_HIP has written nothing.  tq_last_error()
 *    describes the most recent failure of the calling thread.
 *  - Layout of the compressed cache, per (sequence b, KV head h) slot of
 *    `capacity` token positions (capacity a multiple of 32):
 *      k_planes  uint8 [batch][h_kv][ceil(capacity/64)][64*record]: token
 *                records of record = (key_mse_bits + key_qjl)*d/8 +
 *                key_half*d/16 bytes: plane p < key_mse_bits holds bit p of
 *                each coordinate's Lloyd-Max index (coordinate i is bit i%8
 *                of byte i/8); with key_half a half plane of d/16 bytes
 *                follows, bit key_mse_bits of the index of coordinate i
 *                (i mod 32 < 16) at bit position 16*(i/32) + i%32; then the
 *                QJL sign bits (1 = non-negative) in the full-plane order.
 *                The records are stored in blocks of 64 token positions,
 *                interleaved by words: the plane at byte offset o of the
 *                record, s bytes long, fills bytes [64*o, 64*(o+s)) of the
 *                block, and its word w (4 bytes; 2 in the half plane) of the
 *                token at position 64*j + 16*c + n (c < 4, n < 16) is word
 *                4*(4*n + w) + c of that range in block j.
 *      k_norm    [batch][h_kv][capacity] scalar_dtype   |k|
 *      k_rnorm   [batch][h_kv][capacity] scalar_dtype   |r| (QJL keys only)
 *      v_planes  uint32 [batch][h_kv][capacity/32][value_bits][d].  Bit
 *                planes (MSE values; min/max values of width 1 or 3): word
 *                (blk, p, c) holds bit p of the code of token 32*blk+u,
 *                channel c, in bit 8*(u%4) + 4*(u/16) + (u/4)%4.  Packed
 *                codes (min/max values of width b = 2 or 4): word (blk, h, c)
 *                holds the codes of tokens 32*blk + (32/b)*h + i, i < 32/b,
 *                token i's code in bits 8*(i%4) + b*(i/4) .. + b-1.
 *      v_meta    fp16 [batch][h_kv][capacity][d/value_group][2] = (scale, min)
 *                (min/max values only)
 *      v_norm    [batch][h_kv][capacity] scalar_dtype   |v| (MSE values only)
 *  - K/V inputs are [batch][n][h_kv][d] row-major; queries [batch][h_q][d];
 *    the bf16 ring is [batch][ring_cap][h_kv][d] for K and for V.  Query head
 *    hq reads KV head hq / (h_q / h_kv).
 *  - Kernel paths.  Decode runs the int8-MFMA scan for keys of 1, 2 or 3
 *    index bits with or without the QJL bit (or 1.5 / 2.5 with QJL), with
 *    2- or 4-bit min/max values in groups of 32 or 3-bit MSE values (and
 *    2-bit MSE values with 2+1- or 3+1-bit keys), else a VALU scan;
 *    environment variable
 *    TQ_DECODE_PATH=generic forces the VALU scan.  Encode of at most 4 new
 *    tokens per sequence runs a few-token fp32 kernel (keys and MSE values in
 *    one launch for QJL keys of 2 or 3 index bits with 2- or 3-bit MSE
 *    values), else the MFMA rotation kernels; TQ_ENCODE_PATH=small or =mfma
 *    forces one.  All paths compute the same codes up to the boundary window
 *    and the same outputs within rounding.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TQ_OK = 0,
  TQ_ERR_INVALID = -1,     /* bad pointer, size or combination of arguments     */
  TQ_ERR_UNSUPPORTED = -2, /* valid but not built (e.g. head_dim other than 128) */
  TQ_ERR_CAPACITY = -3,    /* a write would land beyond the cache capacity      */
  TQ_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required        */
  TQ_ERR_HIP = -5          /* a HIP launch or API call failed                   */
};

enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 };    /* element types               */
enum { TQ_V_MINMAX = 0, TQ_V_MSE = 1 };          /* value codes                 */
enum { TQ_BYTES_DATA = 0, TQ_BYTES_PARAMS = 1, TQ_BYTES_RING = 2 };

#define TQ_MAX_LEVELS 16 /* 2^4: largest codebook */

/* Quantizer layout.  Only head_dim = 128 is built. */
typedef struct tq_layout {
  int32_t head_dim;     /* d                                                   */
  int32_t key_mse_bits; /* 1..4: Lloyd-Max bits per key coordinate (b-1 of a
                           TurboQuantProd(b) key)                              */
  int32_t key_qjl;      /* 1: one QJL sign bit per coordinate plus |r|; 0: none */
  int32_t value_kind;   /* TQ_V_MINMAX | TQ_V_MSE                              */
  int32_t value_bits;   /* 1..4                                                */
  int32_t value_group;  /* min/max group of consecutive channels; divides d    */
  int32_t scalar_dtype; /* TQ_F32 | TQ_F16: storage of |k|, |r| and |v|        */
  int32_t key_half;     /* 0, or 1: fractional key width key_mse_bits + 1/2;
                           the rotated coordinates i with i mod 32 < 16 use a
                           (key_mse_bits + 1)-bit Lloyd-Max code (page
                           "TurboQuant — ...", sections "Ý tưởng cốt lõi" and
                           "Ý nghĩa thực tế": 2.5 and 3.5 bits per channel).
                           Requires key_qjl = 1 and key_mse_bits 1 or 2, so
                           TurboQuantProd(2.5) and TurboQuantProd(3.5).       */
} tq_layout;

/* Per-layer parameters.  pi, s and derived are device pointers; the codebook
 * tables are host values copied into each launch. */
typedef struct tq_params {
  const float* pi;      /* [d][d] fp32 row-major orthogonal rotation Pi        */
  const float* s;       /* [d][d] fp32 row-major QJL projection S              */
  const void* derived;  /* filled by tq_prepare_params from pi and s           */
  float k_centroids[TQ_MAX_LEVELS];      /* 2^key_mse_bits, ascending          */
  float k_thresholds[TQ_MAX_LEVELS - 1]; /* 2^key_mse_bits - 1 decision bounds */
  float v_centroids[TQ_MAX_LEVELS];      /* MSE values: 2^value_bits levels    */
  float v_thresholds[TQ_MAX_LEVELS - 1];
  float k_centroids_hi[TQ_MAX_LEVELS];   /* key_half: the (key_mse_bits + 1)-bit
                                            table of the half-bit coordinates */
  float k_thresholds_hi[TQ_MAX_LEVELS - 1];
} tq_params;

/* Compressed cache: device planes as described above. */
typedef struct tq_cache {
  uint8_t* k_planes;
  void* k_norm;
  void* k_rnorm;
  uint32_t* v_planes;
  uint16_t* v_meta;
  void* v_norm;
  int32_t batch;
  int32_t num_kv_heads;
  int64_t capacity;
} tq_cache;

/* Lloyd-Max codebook for one coordinate of a randomly rotated unit vector in
 * dimension d: the law with density proportional to (1-x^2)^((d-3)/2) on
 * [-1,1] (page "TurboQuant — ...", section "Ý tưởng cốt lõi": concentrated
 * Beta law, one MSE-optimal scalar quantizer).  Solved in double precision,
 * written as fp32: centroids_host[2^bits] ascending and thresholds_host
 * [2^bits - 1] midpoints.  Host only.  Errors: TQ_ERR_INVALID for d < 3,
 * bits outside 1..4 or NULL outputs. */
int tq_make_codebook(int32_t d, int32_t bits, float* centroids_host, float* thresholds_host);

/* Bytes of the cache (page "turboquant/audit_claims.py", AUDIT 1 accounting).
 * what = TQ_BYTES_DATA: quantized tensors for n_tokens tokens of every
 * (sequence, KV head); TQ_BYTES_PARAMS: Pi and S in fp32 plus the fp32
 * codebook tables (centroids, cell edges, decision thresholds); TQ_BYTES_RING:
 * the bf16 K and V ring of ring_cap tokens.  Returns the count, or a negative
 * TQ_ERR_* code. */
int64_t tq_memory_bytes(const tq_layout* layout, int32_t batch, int32_t num_kv_heads,
                        int64_t n_tokens, int32_t ring_cap, int32_t what);

/* Size of the buffer tq_prepare_params fills for head dimension d. */
size_t tq_params_derived_bytes(int32_t d);

/* Derive, on the device, the per-layer operands the kernels use from Pi and
 * S: bf16 hi/lo splits of Pi and of S Pi^T (the QJL projection of AUDIT 3 of
 * page "turboquant/audit_claims.py" expressed on the rotated residual, since
 * Pi is orthogonal) for the encode, and fp32 Pi^T and S^T for the decode's
 * query rotation and sketch (page "TurboQuant — ...", section "Tại sao nó
 * hoạt động": the query is rotated, the keys never are).  Run once per layer
 * and whenever pi or s change; tq_encode_kv and tq_decode_attn read
 * params->derived.  derived must hold tq_params_derived_bytes(d) bytes
 * (256 KiB at d = 128).  Errors: TQ_ERR_UNSUPPORTED for a d other than 128
 * that is a positive multiple of 32, else TQ_ERR_INVALID for a bad d, a NULL
 * pointer or a derived_bytes below that size. */
int tq_prepare_params(int32_t d, const float* pi, const float* s, void* derived,
                      size_t derived_bytes, void* stream);

/* Encode (page "TurboQuant — ...", section "Ý tưởng cốt lõi"; page
 * "turboquant/audit_claims.py", AUDIT 1 for the value code and AUDIT 3 for
 * TurboQuantProd) n_new tokens of every sequence and KV head into the cache
 * at token positions dst_pos_host[b] .. dst_pos_host[b] + n_new - 1.  k, v:
 * [batch][n_new][h_kv][d] in in_dtype (TQ_F32 or TQ_BF16).  Writes the key
 * planes and norms and the value planes and scalars of those positions only;
 * other positions of a shared 32-token value block are preserved.  Errors:
 * TQ_ERR_CAPACITY when a position exceeds capacity; TQ_ERR_INVALID on NULL or
 * inconsistent pointers. */
int tq_encode_kv(const tq_layout* layout, const tq_params* params, const void* k,
                 const void* v, int32_t in_dtype, int64_t n_new, const int64_t* dst_pos_host,
                 const tq_cache* cache, void* stream);

/* Append (page "turboquant/audit_claims.py", AUDIT 1: the store keeps the
 * most recent tokens uncompressed) one token per sequence to the bf16 ring at position n_ring_host[b]
 * (which must be < ring_cap), rounding to bf16.  k_new, v_new:
 * [batch][1][h_kv][d] in in_dtype (TQ_F32 or TQ_BF16). */
int tq_ring_append(const void* k_new, const void* v_new, int32_t in_dtype, int32_t batch,
                   int32_t num_kv_heads, int32_t head_dim, void* ring_k, void* ring_v,
                   int32_t ring_cap, const int32_t* n_ring_host, void* stream);

/* Workspace bytes tq_decode_attn needs for these sizes (max_tokens = the
 * largest compressed length of any sequence). */
size_t tq_decode_workspace_bytes(const tq_layout* layout, int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int64_t max_tokens);

/* One decode step (page "03. Results & Benchmarks", sections "Latency
 * Benchmarks" and "Next Steps": scores, QJL correction, online softmax and
 * value accumulation fused over the compressed cache; page "TurboQuant —
 * ...", section "Tại sao nó hoạt động" for the rotated query): for every
 * sequence b and query head hq, attention of
 * q[b][hq] over the n_compressed_host[b] compressed tokens of KV head
 * hq / (h_q / h_kv) and the first n_ring_host[b] ring tokens, with scores
 * softmax_scale * <q, k>.  out: [batch][h_q][d] fp32.  q_dtype: TQ_F32 or
 * TQ_BF16.  ring_k/ring_v may be NULL when ring_cap is 0.  A sequence with no
 * token at all gets a zero output.  params->derived must have been filled by
 * tq_prepare_params.  Errors: TQ_ERR_INVALID for a NULL derived buffer or
 * inconsistent sizes, TQ_ERR_WORKSPACE when workspace_bytes is below
 * tq_decode_workspace_bytes. */
int tq_decode_attn(const tq_layout* layout, const tq_params* params, const void* q,
                   int32_t q_dtype, int32_t num_q_heads, const tq_cache* cache,
                   const int64_t* n_compressed_host, const void* ring_k, const void* ring_v,
                   int32_t ring_cap, const int32_t* n_ring_host, float softmax_scale, float* out,
                   void* workspace, size_t workspace_bytes, void* stream);

/* One decode step with the ring append fused in (page
 * "turboquant/audit_claims.py", AUDIT 1: the store keeps the most recent
 * tokens uncompressed; page "03. Results & Benchmarks", section "Latency
 * Benchmarks": one pass per step).  The result equals tq_ring_append of
 * (k_new, v_new) at ring positions n_ring_host[b], followed by tq_decode_attn
 * with n_ring_host[b] + 1 ring tokens.  The append is done by the decode's own
 * query-preparation kernel, with no launch of its own.  k_new, v_new:
 * [batch][1][h_kv][d] in new_dtype (TQ_F32 or TQ_BF16), rounded to bf16 in the
 * ring.  ring_k, ring_v: the caller's bf16 ring [batch][ring_cap][h_kv][d],
 * written at those positions and read for attention.  n_ring_host holds the
 * ring lengths before the append; the caller advances them by one after the
 * call.  One query per sequence; q, out, workspace and the other arguments as
 * tq_decode_attn.  Errors as tq_decode_attn, plus TQ_ERR_INVALID for a NULL
 * k_new, v_new, ring buffer or n_ring_host, a bad new_dtype or ring_cap 0,
 * and TQ_ERR_CAPACITY when n_ring_host[b] + 1 exceeds ring_cap.  A failed
 * check writes nothing. */
int tq_decode_attn_append(const tq_layout* layout, const tq_params* params, const void* q, int32_t q_dtype,
                          int32_t num_q_heads, const tq_cache* cache, const int64_t* n_compressed_host,
                          const void* k_new, const void* v_new, int32_t new_dtype, void* ring_k, void* ring_v,
                          int32_t ring_cap, const int32_t* n_ring_host, float softmax_scale, float* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Multi-query decode (page "turboquant/audit_claims.py", AUDIT 4: the
 * (H_kv, G, T, N) score layout with T query positions per step): num_queries
 * = T queries per sequence, for speculative verification or chunked prefill
 * over the same cache.  q: [batch][T][h_q][d] in q_dtype; out: [batch][T]
 * [h_q][d] fp32.  The T queries are the sequence's last T positions, already
 * in the cache (compressed or ring): with the keys of a sequence ordered as
 * its n_compressed_host[b] compressed tokens followed by its n_ring_host[b]
 * ring tokens, query t sees every key except the last T - 1 - t of that order
 * (causal among the new positions).  A query that sees no key gets a zero
 * output.  Up to 8 (query, head) pairs per KV head share one pass over the
 * compressed cache; larger T * (h_q / h_kv) takes several passes.  workspace
 * must hold tq_decode_workspace_bytes_multi bytes; other arguments and errors
 * as tq_decode_attn, plus TQ_ERR_INVALID for num_queries < 1.  With T = 1 it
 * is tq_decode_attn. */
size_t tq_decode_workspace_bytes_multi(const tq_layout* layout, int32_t batch, int32_t num_q_heads,
                                       int32_t num_kv_heads, int64_t max_tokens, int32_t num_queries);
int tq_decode_attn_multi(const tq_layout* layout, const tq_params* params, const void* q,
                         int32_t q_dtype, int32_t num_q_heads, int32_t num_queries, const tq_cache* cache,
                         const int64_t* n_compressed_host, const void* ring_k, const void* ring_v,
                         int32_t ring_cap, const int32_t* n_ring_host, float softmax_scale, float* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device scratch of tq_decode_attn_noalloc: 32 MiB, the
 * workspace of up to 64 sequences per launch group with 32 KV heads of 8
 * query heads each at any length. */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Decode step that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): tq_decode_attn without the workspace arguments.  The
 * workspace lives in a static device array of TQ_NOALLOC_SCRATCH_BYTES bytes
 * that each GPU holds from the library's first use on it until the process
 * ends; the array's device address is looked up once per device, on the first
 * call made with that device current.  Every call on a GPU shares that GPU's
 * array and the array keeps the last call's contents: calls that overlap on
 * one GPU (two streams, two host threads) race, so the caller serialises
 * them.  Nothing needs clearing between calls: every workspace byte a call
 * reads is written earlier in the same call.  q, out and every other argument
 * as tq_decode_attn.  Errors as tq_decode_attn, plus TQ_ERR_WORKSPACE, with
 * nothing launched, when the call needs more workspace than the scratch holds
 * (tq_decode_workspace_bytes for its sizes above TQ_NOALLOC_SCRATCH_BYTES),
 * and TQ_ERR_HIP when the scratch's address cannot be obtained. */
int tq_decode_attn_noalloc(const tq_layout* layout, const tq_params* params, const void* q,
                           int32_t q_dtype, int32_t num_q_heads, const tq_cache* cache,
                           const int64_t* n_compressed_host, const void* ring_k, const void* ring_v,
                           int32_t ring_cap, const int32_t* n_ring_host, float softmax_scale, float* out,
                           void* stream);

/* Measurement hook.  The next launch of `kernel` (TQ_KERNEL_*) made by the
 * calling thread records ev_begin just before it and ev_end just after it on
 * the launch stream (both hipEvent_t created by the caller), so the caller can
 * time that one kernel with hipEventElapsedTime.  The registration is used
 * once; NULL events cancel it.  Errors: TQ_ERR_INVALID for an unknown kernel. */
enum { TQ_KERNEL_DECODE_SCAN = 0, TQ_KERNEL_ENCODE_KEYS = 1, TQ_KERNEL_ENCODE_VALUES = 2 };
int tq_time_next_launch(int32_t kernel, void* ev_begin, void* ev_end);

/* Text of the most recent error of the calling thread ("" if none). */
const char* tq_last_error(void);

/* Library version string. */
const char* tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
