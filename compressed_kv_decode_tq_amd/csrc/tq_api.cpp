// Host side of the C ABI declared in include/tq.h: argument checks, byte
// accounting and launches.  Every check runs before any launch, so a call
// rejected here has enqueued nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>

#include "tq_internal.h"

namespace tq {
int make_codebook(int d, int bits, double* cent, double* thr);  // tq_codebook.cpp
}

namespace {

thread_local char g_err[512] = "";
thread_local tq::TimedLaunch g_timed[3];  // indexed by TQ_KERNEL_*

tq::TimedLaunch take_timed(int kernel) {
  tq::TimedLaunch t = g_timed[kernel];
  g_timed[kernel] = tq::TimedLaunch{};
  return t;
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_layout(const tq_layout* l) {
  if (!l) return fail(TQ_ERR_INVALID, "layout is NULL");
  if (l->head_dim <= 0 || l->head_dim % 32) return fail(TQ_ERR_INVALID, "head_dim must be a positive multiple of 32");
  if (l->head_dim != tq::kD) return fail(TQ_ERR_UNSUPPORTED, "only head_dim 128 is built (got %d)", l->head_dim);
  if (l->key_mse_bits < 1 || l->key_mse_bits > 4) return fail(TQ_ERR_INVALID, "key_mse_bits must be 1..4");
  if (l->key_qjl != 0 && l->key_qjl != 1) return fail(TQ_ERR_INVALID, "key_qjl must be 0 or 1");
  if (l->value_kind != TQ_V_MINMAX && l->value_kind != TQ_V_MSE) return fail(TQ_ERR_INVALID, "bad value_kind");
  if (l->value_bits < 1 || l->value_bits > 4) return fail(TQ_ERR_INVALID, "value_bits must be 1..4");
  if (l->value_kind == TQ_V_MINMAX) {
    if (l->value_group <= 0 || l->head_dim % l->value_group) return fail(TQ_ERR_INVALID, "value_group must divide head_dim");
    if (l->value_group != 16 && l->value_group != 32 && l->value_group != 64)
      return fail(TQ_ERR_UNSUPPORTED, "value_group %d not built (16, 32, 64 are)", l->value_group);
  }
  if (l->scalar_dtype != TQ_F32 && l->scalar_dtype != TQ_F16) return fail(TQ_ERR_INVALID, "scalar_dtype must be TQ_F32 or TQ_F16");
  if (l->key_half != 0 && l->key_half != 1) return fail(TQ_ERR_INVALID, "key_half must be 0 or 1");
  if (l->key_half && (!l->key_qjl || l->key_mse_bits > 2))
    return fail(TQ_ERR_UNSUPPORTED, "key_half is built for QJL keys with key_mse_bits 1 or 2 (2.5 and 3.5 bits)");
  return TQ_OK;
}

int64_t per_token_head_bytes(const tq_layout* l) {
  const int64_t s = l->scalar_dtype == TQ_F32 ? 4 : 2;
  int64_t k = (int64_t)(l->key_mse_bits + l->key_qjl) * l->head_dim / 8 + (int64_t)l->key_half * l->head_dim / 16 +
              s * (1 + l->key_qjl);
  int64_t v = (int64_t)l->value_bits * l->head_dim / 8;
  v += l->value_kind == TQ_V_MINMAX ? (int64_t)(l->head_dim / l->value_group) * 4 : s;
  return k + v;
}

int check_cache(const tq_layout* l, const tq_cache* c) {
  if (!c) return fail(TQ_ERR_INVALID, "cache is NULL");
  if (c->batch <= 0 || c->num_kv_heads <= 0) return fail(TQ_ERR_INVALID, "cache batch and num_kv_heads must be positive");
  if (c->capacity <= 0 || c->capacity % 32) return fail(TQ_ERR_INVALID, "cache capacity must be a positive multiple of 32");
  if (!c->k_planes || !c->k_norm || !c->v_planes) return fail(TQ_ERR_INVALID, "cache k_planes, k_norm and v_planes are required");
  if (l->key_qjl && !c->k_rnorm) return fail(TQ_ERR_INVALID, "cache k_rnorm is required for QJL keys");
  if (l->value_kind == TQ_V_MINMAX && !c->v_meta) return fail(TQ_ERR_INVALID, "cache v_meta is required for min/max values");
  if (l->value_kind == TQ_V_MSE && !c->v_norm) return fail(TQ_ERR_INVALID, "cache v_norm is required for MSE values");
  return TQ_OK;
}

void fill_codebooks(const tq_layout* l, const tq_params* p, float* kc, float* kt, float* vc, float* vt) {
  const int kl = 1 << l->key_mse_bits;
  for (int i = 0; i < 16; ++i) kc[i] = i < kl ? p->k_centroids[i] : 0.f;
  for (int i = 0; i < 15; ++i) kt[i] = i < kl - 1 ? p->k_thresholds[i] : INFINITY;
  const int vl = 1 << l->value_bits;
  const bool mse = l->value_kind == TQ_V_MSE;
  for (int i = 0; i < 16; ++i) vc[i] = (mse && i < vl) ? p->v_centroids[i] : 0.f;
  for (int i = 0; i < 15; ++i) vt[i] = (mse && i < vl - 1) ? p->v_thresholds[i] : INFINITY;
}

// The (key_mse_bits + 1)-bit key table of the half-bit layout (zeros otherwise).
void fill_hi_codebook(const tq_layout* l, const tq_params* p, float* kc, float* kt) {
  const int kl = l->key_half ? 2 << l->key_mse_bits : 0;
  for (int i = 0; i < 16; ++i) kc[i] = i < kl ? p->k_centroids_hi[i] : 0.f;
  for (int i = 0; i < 15; ++i) kt[i] = i < kl - 1 ? p->k_thresholds_hi[i] : INFINITY;
}

// Byte offset of sequence b0 in a [batch][h_kv][capacity]-strided plane with
// `per_token` bytes per token.
inline size_t seq_off(int b0, int h_kv, int64_t cap, size_t per_token) {
  return (size_t)b0 * h_kv * (size_t)cap * per_token;
}

}  // namespace

extern "C" {

const char* tq_last_error(void) { return g_err; }

int tq_time_next_launch(int32_t kernel, void* ev_begin, void* ev_end) {
  g_err[0] = 0;
  if (kernel < 0 || kernel > 2) return fail(TQ_ERR_INVALID, "unknown kernel id %d", kernel);
  g_timed[kernel].begin = (hipEvent_t)ev_begin;
  g_timed[kernel].end = (hipEvent_t)ev_end;
  return TQ_OK;
}

const char* tq_version(void) { return "tq 0.1 gfx950"; }

int tq_make_codebook(int32_t d, int32_t bits, float* centroids_host, float* thresholds_host) {
  g_err[0] = 0;
  if (d < 3) return fail(TQ_ERR_INVALID, "d must be >= 3");
  if (bits < 1 || bits > 4) return fail(TQ_ERR_INVALID, "bits must be 1..4");
  if (!centroids_host || !thresholds_host) return fail(TQ_ERR_INVALID, "output pointers are NULL");
  double c[16], t[15];
  tq::make_codebook(d, bits, c, t);
  const int levels = 1 << bits;
  for (int i = 0; i < levels; ++i) centroids_host[i] = (float)c[i];
  for (int i = 0; i + 1 < levels; ++i) thresholds_host[i] = (float)t[i];
  return TQ_OK;
}

int64_t tq_memory_bytes(const tq_layout* layout, int32_t batch, int32_t num_kv_heads,
                        int64_t n_tokens, int32_t ring_cap, int32_t what) {
  g_err[0] = 0;
  int rc = check_layout(layout);
  if (rc != TQ_OK && rc != TQ_ERR_UNSUPPORTED) return rc;  // byte counts hold for any d
  if (batch < 0 || num_kv_heads < 0 || n_tokens < 0 || ring_cap < 0)
    return fail(TQ_ERR_INVALID, "sizes must be non-negative");
  const int64_t d = layout->head_dim;
  switch (what) {
    case TQ_BYTES_DATA:
      return per_token_head_bytes(layout) * batch * num_kv_heads * n_tokens;
    case TQ_BYTES_PARAMS: {
      auto tables = [](int bits) { const int64_t L = 1 << bits; return 4 * (L + (L + 1) + (L - 1)); };
      int64_t p = 2 * d * d * 4 + tables(layout->key_mse_bits);
      if (layout->key_half) p += tables(layout->key_mse_bits + 1);
      if (layout->value_kind == TQ_V_MSE) p += tables(layout->value_bits);
      return p;
    }
    case TQ_BYTES_RING:
      return (int64_t)batch * ring_cap * num_kv_heads * d * 2 * 2;
    default:
      return fail(TQ_ERR_INVALID, "unknown 'what' %d", what);
  }
}

size_t tq_params_derived_bytes(int32_t d) { return d == tq::kD ? tq::kDerivedBytes : 0; }

int tq_prepare_params(int32_t d, const float* pi, const float* s, void* derived,
                      size_t derived_bytes, void* stream) {
  g_err[0] = 0;
  if (d != tq::kD) return fail(d > 0 && d % 32 == 0 ? TQ_ERR_UNSUPPORTED : TQ_ERR_INVALID, "only d = 128 is built");
  if (!pi || !s || !derived) return fail(TQ_ERR_INVALID, "pi, s and derived must be non-NULL");
  if (derived_bytes < tq::kDerivedBytes) return fail(TQ_ERR_INVALID, "derived buffer too small");
  hipError_t e = tq::launch_prepare_params(pi, s, (uint16_t*)derived, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "prepare_params launch");
}

int tq_encode_kv(const tq_layout* layout, const tq_params* params, const void* k, const void* v,
                 int32_t in_dtype, int64_t n_new, const int64_t* dst_pos_host,
                 const tq_cache* cache, void* stream) {
  g_err[0] = 0;
  int rc = check_layout(layout);
  if (rc) return rc;
  if ((rc = check_cache(layout, cache))) return rc;
  if (!params || !params->pi || !params->s || !params->derived)
    return fail(TQ_ERR_INVALID, "params pi, s and derived must be set");
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16) return fail(TQ_ERR_INVALID, "in_dtype must be TQ_F32 or TQ_BF16");
  if (n_new < 0) return fail(TQ_ERR_INVALID, "n_new must be >= 0");
  if (n_new == 0) return TQ_OK;
  if (!k || !v || !dst_pos_host) return fail(TQ_ERR_INVALID, "k, v and dst_pos_host must be non-NULL");
  for (int b = 0; b < cache->batch; ++b) {
    if (dst_pos_host[b] < 0) return fail(TQ_ERR_INVALID, "dst_pos_host[%d] is negative", b);
    if (dst_pos_host[b] + n_new > cache->capacity)
      return fail(TQ_ERR_CAPACITY, "sequence %d: positions up to %lld exceed capacity %lld", b,
                  (long long)(dst_pos_host[b] + n_new), (long long)cache->capacity);
  }
  const int h_kv = cache->num_kv_heads;
  const int64_t cap = cache->capacity;
  const size_t esz = in_dtype == TQ_F32 ? 4 : 2;
  const size_t sz = layout->scalar_dtype == TQ_F32 ? 4 : 2;
  const size_t kpb = tq::key_record_bytes(layout->key_mse_bits, layout->key_qjl, layout->key_half);
  const size_t groups = layout->value_kind == TQ_V_MINMAX ? tq::kD / layout->value_group : 0;
  const bool bf16 = in_dtype == TQ_BF16;
  hipStream_t st = (hipStream_t)stream;

  for (int b0 = 0; b0 < cache->batch; b0 += tq::kMaxSeqPerLaunch) {
    const int nb = std::min(tq::kMaxSeqPerLaunch, cache->batch - b0);
    tq::EncodeArgs a;
    std::memset(&a, 0, sizeof(a));
    const size_t in_off = (size_t)b0 * n_new * h_kv * tq::kD * esz;
    a.k = (const char*)k + in_off;
    a.v = (const char*)v + in_off;
    a.k_planes = cache->k_planes + seq_off(b0, h_kv, tq::key_slot_tokens(cap), kpb);
    a.k_norm = (char*)cache->k_norm + seq_off(b0, h_kv, cap, sz);
    a.k_rnorm = cache->k_rnorm ? (char*)cache->k_rnorm + seq_off(b0, h_kv, cap, sz) : nullptr;
    a.v_planes = (uint32_t*)((char*)cache->v_planes + seq_off(b0, h_kv, cap, (size_t)layout->value_bits * tq::kD / 8));
    a.v_meta = cache->v_meta ? (uint16_t*)((char*)cache->v_meta + seq_off(b0, h_kv, cap, groups * 4)) : nullptr;
    a.v_norm = cache->v_norm ? (char*)cache->v_norm + seq_off(b0, h_kv, cap, sz) : nullptr;
    a.derived = (const uint16_t*)params->derived;
    a.pi = params->pi;
    a.n_new = n_new;
    a.capacity = cap;
    a.batch = nb;
    a.h_kv = h_kv;
    a.scalar_f16 = layout->scalar_dtype == TQ_F16;
    a.value_group = layout->value_group;
    fill_codebooks(layout, params, a.k_cent, a.k_thr, a.v_cent, a.v_thr);
    fill_hi_codebook(layout, params, a.k_cent_hi, a.k_thr_hi);
    int64_t tiles = 0;
    for (int b = 0; b < nb; ++b) {
      const int64_t pos = dst_pos_host[b0 + b];
      a.pos.v[b] = pos;
      a.tile_start.v[b] = tiles;
      tiles += (int64_t)h_kv * (((pos + n_new + 31) >> 5) - (pos >> 5));
    }
    if (tiles > INT32_MAX) return fail(TQ_ERR_UNSUPPORTED, "too many tokens in one call");
    // tile_start has kMaxSeqPerLaunch entries; the kernels stop their search at
    // `batch`, and num_tiles bounds the last sequence.
    a.num_tiles = (int32_t)tiles;
    // few tokens with MSE values: keys and values in one launch, unless a
    // caller asked to time one of the two kernels on its own
    hipError_t e = hipErrorNotSupported;
    if (layout->value_kind == TQ_V_MSE && !g_timed[TQ_KERNEL_ENCODE_KEYS].begin &&
        !g_timed[TQ_KERNEL_ENCODE_VALUES].begin)
      e = tq::launch_encode_small_kv(a, bf16, layout->key_mse_bits, layout->key_qjl, layout->key_half,
                                     layout->value_bits, st);
    if (e != hipErrorNotSupported) {
      if (e != hipSuccess) return hip_fail(e, "encode launch");
      continue;
    }
    e = tq::launch_encode_keys(a, bf16, layout->key_mse_bits, layout->key_qjl, layout->key_half, st,
                               take_timed(TQ_KERNEL_ENCODE_KEYS));
    if (e != hipSuccess) return hip_fail(e, "encode keys launch");
    if (layout->value_kind == TQ_V_MSE)
      e = tq::launch_encode_values_mse(a, bf16, layout->value_bits, st, take_timed(TQ_KERNEL_ENCODE_VALUES));
    else
      e = tq::launch_encode_values_minmax(a, bf16, layout->value_bits, st, take_timed(TQ_KERNEL_ENCODE_VALUES));
    if (e != hipSuccess) return hip_fail(e, "encode values launch");
  }
  return TQ_OK;
}

int tq_ring_append(const void* k_new, const void* v_new, int32_t in_dtype, int32_t batch,
                   int32_t num_kv_heads, int32_t head_dim, void* ring_k, void* ring_v,
                   int32_t ring_cap, const int32_t* n_ring_host, void* stream) {
  g_err[0] = 0;
  if (head_dim != tq::kD) return fail(TQ_ERR_UNSUPPORTED, "only head_dim 128 is built");
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16) return fail(TQ_ERR_INVALID, "in_dtype must be TQ_F32 or TQ_BF16");
  if (batch <= 0 || num_kv_heads <= 0 || ring_cap <= 0) return fail(TQ_ERR_INVALID, "sizes must be positive");
  if (!k_new || !v_new || !ring_k || !ring_v || !n_ring_host) return fail(TQ_ERR_INVALID, "NULL pointer");
  for (int b = 0; b < batch; ++b)
    if (n_ring_host[b] < 0 || n_ring_host[b] >= ring_cap)
      return fail(TQ_ERR_CAPACITY, "sequence %d: ring position %d outside [0, %d)", b, n_ring_host[b], ring_cap);
  const size_t esz = in_dtype == TQ_F32 ? 4 : 2;
  for (int b0 = 0; b0 < batch; b0 += tq::kMaxSeqPerLaunch) {
    const int nb = std::min(tq::kMaxSeqPerLaunch, batch - b0);
    tq::SeqValues nr;
    for (int b = 0; b < nb; ++b) nr.v[b] = n_ring_host[b0 + b];
    const size_t in_off = (size_t)b0 * num_kv_heads * tq::kD * esz;
    const size_t ring_off = (size_t)b0 * ring_cap * num_kv_heads * tq::kD;
    hipError_t e = tq::launch_ring_append((const char*)k_new + in_off, (const char*)v_new + in_off,
                                          in_dtype == TQ_BF16, nb, num_kv_heads,
                                          (uint16_t*)ring_k + ring_off, (uint16_t*)ring_v + ring_off,
                                          ring_cap, nr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ring append launch");
  }
  return TQ_OK;
}

}  // extern "C"

namespace {

// Virtual heads one decode launch handles per KV head: all query heads of a
// KV head for one query per sequence; for several queries, up to kMaxGroup
// (query, head) pairs per launch.
int decode_vgroup(int group, int nq) { return std::min(tq::kMaxGroup, group * nq); }

size_t decode_ws_bytes(int nb, int h_kv, int vg, int64_t max_tokens) {
  const int32_t splits = tq::decode_max_splits(max_tokens, (int64_t)nb * h_kv);
  const size_t rows = (size_t)nb * h_kv * vg;
  const size_t qprep = rows * 2 * tq::kD * 4;
  const size_t part = (size_t)splits * rows * (tq::kD + 2) * 4;
  const size_t base = (qprep + part + 255) & ~(size_t)255;
  return base + tq::mfma_workspace_bytes(nb, h_kv * vg, vg);
}

size_t decode_workspace_bytes_impl(const tq_layout* layout, int32_t batch, int32_t num_q_heads,
                                   int32_t num_kv_heads, int64_t max_tokens, int32_t nq) {
  if (!layout || batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_tokens < 0 || nq <= 0) return 0;
  if (num_q_heads % num_kv_heads) return 0;
  const int nb = std::min(batch, tq::kMaxSeqPerLaunch);
  return decode_ws_bytes(nb, num_kv_heads, decode_vgroup(num_q_heads / num_kv_heads, nq), max_tokens);
}

// One decode call.  With k_new (fused append, nq = 1): the token k_new[b],
// v_new[b] is first written to ring position n_ring_host[b], and attention
// covers n_ring_host[b] + 1 ring tokens.
int decode_attn_impl(const tq_layout* layout, const tq_params* params, const void* q, int32_t q_dtype,
                     int32_t num_q_heads, int32_t nq, const tq_cache* cache, const int64_t* n_compressed_host,
                     const void* ring_k, const void* ring_v, int32_t ring_cap, const int32_t* n_ring_host,
                     float softmax_scale, float* out, void* workspace, size_t workspace_bytes, void* stream,
                     const void* k_new = nullptr, const void* v_new = nullptr, int32_t new_dtype = 0,
                     bool noalloc = false) {
  g_err[0] = 0;
  const bool append = k_new != nullptr || v_new != nullptr;
  if (append) {
    if (!k_new || !v_new) return fail(TQ_ERR_INVALID, "k_new and v_new must both be non-NULL");
    if (new_dtype != TQ_F32 && new_dtype != TQ_BF16) return fail(TQ_ERR_INVALID, "new_dtype must be TQ_F32 or TQ_BF16");
    if (ring_cap <= 0) return fail(TQ_ERR_INVALID, "the fused append needs a ring (ring_cap > 0)");
    if (!ring_k || !ring_v || !n_ring_host) return fail(TQ_ERR_INVALID, "ring buffers and n_ring_host required");
    if (nq != 1) return fail(TQ_ERR_INVALID, "the fused append takes one query per sequence");
  }
  int rc = check_layout(layout);
  if (rc) return rc;
  if ((rc = check_cache(layout, cache))) return rc;
  if (!params || !params->pi || !params->s) return fail(TQ_ERR_INVALID, "params pi and s must be set");
  if (!params->derived) return fail(TQ_ERR_INVALID, "params.derived must be filled by tq_prepare_params");
  if (!q || !out || !n_compressed_host) return fail(TQ_ERR_INVALID, "q, out and n_compressed_host must be non-NULL");
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_ERR_INVALID, "q_dtype must be TQ_F32 or TQ_BF16");
  if (nq <= 0) return fail(TQ_ERR_INVALID, "num_queries must be positive");
  const int h_kv = cache->num_kv_heads;
  if (num_q_heads <= 0 || num_q_heads % h_kv) return fail(TQ_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / h_kv;
  if (group > tq::kMaxGroup) return fail(TQ_ERR_UNSUPPORTED, "at most %d query heads per KV head are built", tq::kMaxGroup);
  if (!std::isfinite(softmax_scale)) return fail(TQ_ERR_INVALID, "softmax_scale must be finite");
  if (ring_cap < 0) return fail(TQ_ERR_INVALID, "ring_cap must be >= 0");
  if (ring_cap > 0 && (!ring_k || !ring_v || !n_ring_host)) return fail(TQ_ERR_INVALID, "ring buffers and n_ring_host required when ring_cap > 0");
  int64_t max_tokens = 0;
  for (int b = 0; b < cache->batch; ++b) {
    if (n_compressed_host[b] < 0 || n_compressed_host[b] > cache->capacity)
      return fail(TQ_ERR_CAPACITY, "sequence %d: n_compressed %lld outside [0, capacity]", b, (long long)n_compressed_host[b]);
    if (ring_cap > 0 && (n_ring_host[b] < 0 || n_ring_host[b] + (append ? 1 : 0) > ring_cap))
      return fail(TQ_ERR_CAPACITY, "sequence %d: n_ring %d%s outside [0, ring_cap]", b, n_ring_host[b],
                  append ? " + 1 appended" : "");
    if (ring_cap > 0 && n_ring_host[b] + (append ? 1 : 0) > tq::kMaxRing)
      return fail(TQ_ERR_UNSUPPORTED, "sequence %d: more than %d ring tokens", b, tq::kMaxRing);
    max_tokens = std::max<int64_t>(max_tokens, n_compressed_host[b]);
  }
  const size_t need = decode_workspace_bytes_impl(layout, cache->batch, num_q_heads, h_kv, max_tokens, nq);
  if (noalloc) {
    // the static scratch: sizes beyond it are refused before the device is touched
    if (need > TQ_NOALLOC_SCRATCH_BYTES)
      return fail(TQ_ERR_WORKSPACE, "this call needs %zu bytes of workspace; the static scratch of "
                  "tq_decode_attn_noalloc holds %zu", need, (size_t)TQ_NOALLOC_SCRATCH_BYTES);
    hipError_t e = tq::noalloc_scratch(&workspace, &workspace_bytes);
    if (e != hipSuccess) return hip_fail(e, "static decode scratch address");
  }
  if (!workspace || workspace_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);

  const int64_t cap = cache->capacity;
  const size_t sz = layout->scalar_dtype == TQ_F32 ? 4 : 2;
  const size_t kpb = tq::key_record_bytes(layout->key_mse_bits, layout->key_qjl, layout->key_half);
  const size_t groups = layout->value_kind == TQ_V_MINMAX ? tq::kD / layout->value_group : 0;
  const size_t qsz = q_dtype == TQ_F32 ? 4 : 2;
  const int vg_max = decode_vgroup(group, nq);
  const int nvirt = group * nq;
  float kc[16], kt[15], vc[16], vt[15];
  fill_codebooks(layout, params, kc, kt, vc, vt);
  for (int b0 = 0; b0 < cache->batch; b0 += tq::kMaxSeqPerLaunch) {
    const int nb = std::min(tq::kMaxSeqPerLaunch, cache->batch - b0);
    tq::DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int b = 0; b < nb; ++b) {
      a.n_comp.v[b] = n_compressed_host[b0 + b];
      a.n_ring.v[b] = ring_cap > 0 ? n_ring_host[b0 + b] + (append ? 1 : 0) : 0;
    }
    const size_t new_off = (size_t)b0 * h_kv * tq::kD * (new_dtype == TQ_F32 ? 4 : 2);
    tq::decode_split(max_tokens, (int64_t)std::min(cache->batch, tq::kMaxSeqPerLaunch) * h_kv, &a.splits, &a.split_len);
    a.q = (const char*)q + (size_t)b0 * nq * num_q_heads * tq::kD * qsz;
    a.k_planes = cache->k_planes + seq_off(b0, h_kv, tq::key_slot_tokens(cap), kpb);
    a.k_norm = (const char*)cache->k_norm + seq_off(b0, h_kv, cap, sz);
    a.k_rnorm = cache->k_rnorm ? (const char*)cache->k_rnorm + seq_off(b0, h_kv, cap, sz) : nullptr;
    a.v_planes = (const uint32_t*)((const char*)cache->v_planes + seq_off(b0, h_kv, cap, (size_t)layout->value_bits * tq::kD / 8));
    a.v_meta = cache->v_meta ? (const uint16_t*)((const char*)cache->v_meta + seq_off(b0, h_kv, cap, groups * 4)) : nullptr;
    a.v_norm = cache->v_norm ? (const char*)cache->v_norm + seq_off(b0, h_kv, cap, sz) : nullptr;
    a.pi = params->pi;
    a.s = params->s;
    a.mat_t = reinterpret_cast<const float*>(static_cast<const char*>(params->derived) + tq::kOffPiT);
    const size_t ring_off = (size_t)b0 * ring_cap * h_kv * tq::kD;
    a.ring_k = ring_cap > 0 ? (const uint16_t*)ring_k + ring_off : nullptr;
    a.ring_v = ring_cap > 0 ? (const uint16_t*)ring_v + ring_off : nullptr;
    if (append) {
      a.app_k = (const char*)k_new + new_off;
      a.app_v = (const char*)v_new + new_off;
      a.app_ring_k = const_cast<uint16_t*>(a.ring_k);
      a.app_ring_v = const_cast<uint16_t*>(a.ring_v);
      a.app_bf16 = new_dtype == TQ_BF16;
    }
    a.out = out + (size_t)b0 * nq * num_q_heads * tq::kD;
    // workspace: qprep and partials sized for vg_max virtual heads per KV head
    const size_t rows = (size_t)nb * h_kv * vg_max;
    a.qprep = (float*)workspace;
    a.partial = (float*)((char*)workspace + rows * 2 * tq::kD * 4);
    const size_t base_ws = rows * 2 * tq::kD * 4 + (size_t)a.splits * rows * (tq::kD + 2) * 4;
    a.qdig = (int8_t*)((char*)workspace + ((base_ws + 255) & ~(size_t)255));
    a.qconst = (float*)((char*)a.qdig + (size_t)nb * h_kv * ((vg_max + 3) / 4) * 5 * 2 * 64 * 16);
    a.capacity = cap;
    a.batch = nb;
    a.h_q = num_q_heads;
    a.h_kv = h_kv;
    a.nq = nq;
    a.qgroup = group;
    a.q_bf16 = q_dtype == TQ_BF16;
    a.scalar_f16 = layout->scalar_dtype == TQ_F16;
    a.value_group = layout->value_group;
    a.ring_cap = ring_cap;
    a.scale = softmax_scale;
    std::memcpy(a.k_cent, kc, sizeof(kc));
    std::memcpy(a.v_cent, vc, sizeof(vc));
    const bool vmse = layout->value_kind == TQ_V_MSE;
    const int kpl = tq::plane_expansion(kc, layout->key_mse_bits, a.key_w, &a.key_cst);
    const int vpl = vmse ? tq::plane_expansion(vc, layout->value_bits, a.val_w, &a.val_cst) : 0;
    const char* path = std::getenv("TQ_DECODE_PATH");
    const bool generic_only = path && std::strcmp(path, "generic") == 0;
    // half-bit keys run on the MFMA scan only: its planes come from the
    // (key_mse_bits + 1)-bit table, the base table's weights cover its planes
    int kbits = layout->key_mse_bits, kplanes = kpl;
    if (layout->key_half) {
      float kch[16], kth[15];
      fill_hi_codebook(layout, params, kch, kth);
      kplanes = tq::plane_expansion(kch, layout->key_mse_bits + 1, a.key_w_hi, &a.key_cst_hi);
      kbits = layout->key_mse_bits + 1;
      a.key_half = 1;
      if (generic_only || kpl == 0 || kplanes == 0 || (vmse && vpl == 0))
        return fail(TQ_ERR_UNSUPPORTED, "half-bit keys need the MFMA scan (antisymmetric key and value tables)");
    }
    // one set of launches (q-prep, scan, combine) per group of virtual heads;
    // each pass reads the compressed cache once
    for (int vbase = 0; vbase < nvirt; vbase += vg_max) {
      a.vbase = vbase;
      a.group = std::min(vg_max, nvirt - vbase);
      const tq::TimedLaunch tl = take_timed(TQ_KERNEL_DECODE_SCAN);
      hipError_t e = hipErrorNotSupported;
      if (!generic_only && kpl > 0 && (!vmse || vpl > 0))
        e = tq::launch_decode_mfma(a, kbits, layout->key_qjl, vmse, layout->value_bits, kplanes,
                                   vpl, (hipStream_t)stream, tl);
      if (e == hipErrorNotSupported && layout->key_half)
        return fail(TQ_ERR_UNSUPPORTED, "half-bit keys: this value layout or head group has no MFMA scan");
      if (e == hipErrorNotSupported && append) {
        // the generic path appends with its own launch (the write is idempotent)
        tq::SeqValues pos;
        for (int b = 0; b < nb; ++b) pos.v[b] = n_ring_host[b0 + b];
        e = tq::launch_ring_append(a.app_k, a.app_v, a.app_bf16, nb, h_kv, a.app_ring_k, a.app_ring_v, ring_cap,
                                   pos, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "ring append launch");
        e = hipErrorNotSupported;
      }
      if (e == hipErrorNotSupported)
        e = tq::launch_decode(a, layout->key_mse_bits, layout->key_qjl, vmse, layout->value_bits,
                              (hipStream_t)stream, tl);
      if (e != hipSuccess) return hip_fail(e, "decode launch");
    }
  }
  return TQ_OK;
}

}  // namespace

extern "C" {

size_t tq_decode_workspace_bytes(const tq_layout* layout, int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int64_t max_tokens) {
  return decode_workspace_bytes_impl(layout, batch, num_q_heads, num_kv_heads, max_tokens, 1);
}

size_t tq_decode_workspace_bytes_multi(const tq_layout* layout, int32_t batch, int32_t num_q_heads,
                                       int32_t num_kv_heads, int64_t max_tokens, int32_t num_queries) {
  return decode_workspace_bytes_impl(layout, batch, num_q_heads, num_kv_heads, max_tokens, num_queries);
}

int tq_decode_attn(const tq_layout* layout, const tq_params* params, const void* q,
                   int32_t q_dtype, int32_t num_q_heads, const tq_cache* cache,
                   const int64_t* n_compressed_host, const void* ring_k, const void* ring_v,
                   int32_t ring_cap, const int32_t* n_ring_host, float softmax_scale, float* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return decode_attn_impl(layout, params, q, q_dtype, num_q_heads, 1, cache, n_compressed_host, ring_k, ring_v,
                          ring_cap, n_ring_host, softmax_scale, out, workspace, workspace_bytes, stream);
}

int tq_decode_attn_append(const tq_layout* layout, const tq_params* params, const void* q, int32_t q_dtype,
                          int32_t num_q_heads, const tq_cache* cache, const int64_t* n_compressed_host,
                          const void* k_new, const void* v_new, int32_t new_dtype, void* ring_k, void* ring_v,
                          int32_t ring_cap, const int32_t* n_ring_host, float softmax_scale, float* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new) {
    g_err[0] = 0;
    return fail(TQ_ERR_INVALID, "k_new and v_new must both be non-NULL");
  }
  return decode_attn_impl(layout, params, q, q_dtype, num_q_heads, 1, cache, n_compressed_host, ring_k, ring_v,
                          ring_cap, n_ring_host, softmax_scale, out, workspace, workspace_bytes, stream, k_new,
                          v_new, new_dtype);
}

int tq_decode_attn_noalloc(const tq_layout* layout, const tq_params* params, const void* q,
                           int32_t q_dtype, int32_t num_q_heads, const tq_cache* cache,
                           const int64_t* n_compressed_host, const void* ring_k, const void* ring_v,
                           int32_t ring_cap, const int32_t* n_ring_host, float softmax_scale, float* out,
                           void* stream) {
  return decode_attn_impl(layout, params, q, q_dtype, num_q_heads, 1, cache, n_compressed_host, ring_k, ring_v,
                          ring_cap, n_ring_host, softmax_scale, out, nullptr, 0, stream, nullptr, nullptr, 0,
                          true);
}

int tq_decode_attn_multi(const tq_layout* layout, const tq_params* params, const void* q,
                         int32_t q_dtype, int32_t num_q_heads, int32_t num_queries, const tq_cache* cache,
                         const int64_t* n_compressed_host, const void* ring_k, const void* ring_v,
                         int32_t ring_cap, const int32_t* n_ring_host, float softmax_scale, float* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return decode_attn_impl(layout, params, q, q_dtype, num_q_heads, num_queries, cache, n_compressed_host, ring_k,
                          ring_v, ring_cap, n_ring_host, softmax_scale, out, workspace, workspace_bytes, stream);
}

}  // extern "C"
