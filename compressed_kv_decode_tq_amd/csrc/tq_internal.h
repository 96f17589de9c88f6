// Internal declarations shared by the host entry points and the HIP kernels of
// libtq.  Nothing here is part of the C ABI (include/tq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

constexpr int kD = 128;            // head dimension every kernel is built for
constexpr int kMaxSeqPerLaunch = 64; // per-sequence host values travel in kernel arguments
constexpr int kMaxGroup = 8;       // query heads per KV head handled by one decode work-group
constexpr int kMaxRing = 128;      // ring tokens attended per sequence

// Byte offsets of the operands tq_prepare_params derives from Pi and S.
//   pi_hi/pi_lo : bf16 [128][128] row-major, Pi = pi_hi + pi_lo + O(2^-17 |Pi|)
//   sp_hi/sp_lo : bf16 [128][128], S' = S Pi^T with its columns permuted into the
//                 order in which the encode kernel holds the rotated residual
//                 (see sp_column)
//   pi_t/s_t    : fp32 [128][128], Pi^T and S^T (column j of Pi is row j), so the
//                 decode's query rotation reads them coalesced
constexpr size_t kOffPiHi = 0;
constexpr size_t kOffPiLo = kOffPiHi + kD * kD * 2;
constexpr size_t kOffSpHi = kOffPiLo + kD * kD * 2;
constexpr size_t kOffSpLo = kOffSpHi + kD * kD * 2;
constexpr size_t kOffPiT = kOffSpLo + kD * kD * 2;
constexpr size_t kOffST = kOffPiT + kD * kD * 4;
constexpr size_t kDerivedBytes = kOffST + kD * kD * 4;

// Bytes of one token's key record: full planes, the half plane of the
// fractional layout (coordinates i with i mod 32 < 16), the QJL plane.
inline size_t key_record_bytes(int mse_bits, int qjl, int half) {
  return (size_t)(mse_bits + qjl) * (kD / 8) + (size_t)half * (kD / 16);
}

// Key planes are stored in blocks of 64 token positions; a slot holds
// ceil(capacity / 64) blocks.  Inside a block every plane of the record (at
// byte offset o of the record: full planes of 16 bytes, the half plane of 8)
// takes 64 times its size from byte 64 o, and word w of token u = 16 c + n
// (c < 4, n < 16) of the block (coordinates 32 w .. 32 w + 31: 4 bytes, 2 in
// the half plane) sits at word index 4 (4 n + w) + c of that region.  The
// decode scan's lane (w, n) then finds the words of its four 16-token column
// tiles side by side, and a wave reads each plane of a 64-token chunk as one
// contiguous block.
__host__ __device__ constexpr int64_t key_slot_tokens(int64_t capacity) { return (capacity + 63) / 64 * 64; }
__host__ __device__ constexpr size_t key_word_offset(int64_t t, size_t rec, size_t plane_off, int w, int wbytes) {
  return (size_t)(t >> 6) * 64 * rec + plane_off * 64 + (size_t)((((int)(t & 15) << 2) + w) * 4 + (int)((t >> 4) & 3)) * wbytes;
}

// Column of S' that the encode kernel's second GEMM meets at contraction index
// k.  The first GEMM leaves, in lane group g of a 16x16x32 MFMA, the rotated
// coordinates 16*rt + 4*g + r (row tile rt, accumulator r); the kernel feeds
// them back as the B operand of k-step ks = rt/2 without moving data, so
// contraction index k = 32*ks + 8*g + e holds coordinate 16*(2*ks + e/4) + 4*g + e%4.
__host__ __device__ constexpr int sp_column(int k) {
  return 16 * (2 * (k / 32) + (k % 8) / 4) + 4 * ((k % 32) / 8) + (k % 4);
}

// Per-sequence values for one launch (at most kMaxSeqPerLaunch sequences).
struct SeqValues {
  int64_t v[kMaxSeqPerLaunch];
};

struct EncodeArgs {
  const void* k;         // [batch][n_new][h_kv][d]
  const void* v;
  uint8_t* k_planes;
  void* k_norm;
  void* k_rnorm;
  uint32_t* v_planes;
  uint16_t* v_meta;
  void* v_norm;
  const uint16_t* derived;  // bf16 matrices at the kOff* offsets (in elements: /2)
  const float* pi;          // fp32 Pi, row-major [d][d] (the few-token encode)
  int64_t n_new;
  int64_t capacity;
  int32_t batch;          // sequences in this launch
  int32_t h_kv;
  int32_t scalar_f16;     // 1: scalars stored as fp16
  int32_t value_group;
  int32_t num_tiles;      // (sequence, head, 32-token block) tiles of this launch
  int32_t blocks_per_seq_head_max;
  float k_cent[16];
  float k_thr[15];
  float v_cent[16];
  float v_thr[15];
  float k_cent_hi[16];    // key_half: table of the half-bit coordinates
  float k_thr_hi[15];
  SeqValues pos;          // first destination position per sequence
  SeqValues tile_start;   // prefix count of tiles per sequence (tile_start.v[batch] = total)
};

struct DecodeArgs {
  const void* q;          // [batch][nq][h_q][d]
  const uint8_t* k_planes;
  const void* k_norm;
  const void* k_rnorm;
  const uint32_t* v_planes;
  const uint16_t* v_meta;
  const void* v_norm;
  const float* pi;        // fp32 [d][d]
  const float* s;
  const float* mat_t;     // fp32 Pi^T then S^T ([2][d][d], from the derived buffer)
  const uint16_t* ring_k; // bf16 [batch][ring_cap][h_kv][d]
  const uint16_t* ring_v;
  float* out;             // [batch][nq][h_q][d]
  float* qprep;           // workspace: [batch][h_kv][group][2][d] fp32 (Pi q, S q)
  float* partial;         // workspace: [splits][batch][h_kv][group][d + 2] (m, l, acc)
  int64_t capacity;
  int32_t batch;
  int32_t h_q;
  int32_t h_kv;
  int32_t group;          // virtual heads per KV head in this launch (<= kMaxGroup)
  int32_t nq;             // queries per sequence (T)
  int32_t qgroup;         // query heads per KV head (h_q / h_kv)
  int32_t vbase;          // first virtual head of this launch
  int32_t q_bf16;
  int32_t scalar_f16;
  int32_t value_group;
  int32_t ring_cap;
  int32_t splits;
  int32_t split_len;      // tokens per split (multiple of 64)
  float scale;            // softmax scale tau
  float k_cent[16];
  float v_cent[16];
  // Bit-plane expansion of the codebooks (MFMA path): c[idx] = cst + sum_p w[p] * plane_p(idx)
  // with planes bit0, bit1, bit2, bit0^bit1^bit2 (see plane_expansion).
  float key_w[4];
  float key_cst;
  float key_w_hi[4];      // key_half: expansion of the half-bit coordinates' table
  float key_cst_hi;
  int32_t key_half;
  float val_w[4];
  float val_cst;
  int8_t* qdig;           // workspace: query digit operands of the MFMA scan
  float* qconst;          // workspace: [batch][h_kv][group][4] per-head score constants
  SeqValues n_comp;
  SeqValues n_ring;
  // Fused ring append (single query): the new token of sequence b and KV head
  // h (app_k, app_v: [batch][h_kv][d], bf16 if app_bf16 else fp32) goes to
  // ring position n_ring[b] - 1 before attention; the MFMA q-prep kernel
  // writes it.  NULL app_k: no append.
  const void* app_k;
  const void* app_v;
  uint16_t* app_ring_k;
  uint16_t* app_ring_v;
  int32_t app_bf16;
};

// Multi-query decode.  The nq queries of a sequence against one KV head form
// nq * qgroup virtual heads v = t * qgroup + g (query t, query head
// h * qgroup + g); one set of launches handles `group` of them from vbase on.
// With nq = 1 and vbase = 0 a virtual head is the query head itself.
__host__ __device__ inline void virtual_head(const DecodeArgs& a, int h, int gq, int& t, int& hq) {
  const int v = a.vbase + gq;
  t = v / a.qgroup;
  hq = h * a.qgroup + v % a.qgroup;
}
// Keys hidden from query t: the last nq - 1 - t of the sequence's
// compressed-then-ring order, taken from the ring first.
__host__ __device__ inline void hidden_keys(const DecodeArgs& a, int t, int nr, int& hide_c, int& hide_r) {
  const int hd = a.nq - 1 - t;
  hide_r = hd < nr ? hd : nr;
  hide_c = hd - hide_r;
}
// Row of (sequence b, KV head h, virtual head gq of the launch) in the
// workspace arrays, and of (sequence b, query t, query head hq) in q and out.
__host__ __device__ inline size_t ws_row(const DecodeArgs& a, int b, int h, int gq) {
  return ((size_t)b * a.h_kv + h) * a.group + gq;
}
__host__ __device__ inline size_t q_row(const DecodeArgs& a, int b, int t, int hq) {
  return ((size_t)b * a.nq + t) * a.h_q + hq;
}

// Expansion of a symmetric codebook over bit planes: for idx = sum_k b_k 2^k,
//   c[idx] = cst + sum_p w[p] * plane_p, plane_0..2 = b_0..b_2, plane_3 = b_0^b_1^b_2.
// Returns the number of planes (2^(bits-1)), or 0 when the table is not
// antisymmetric (c[2^b - 1 - i] = -c[i]) to 1e-6 relative, bits > 3, or bits < 1.
int plane_expansion(const float* cent, int bits, float* w, float* cst);

// Events recorded around one kernel launch (both null: none).
struct TimedLaunch {
  hipEvent_t begin = nullptr;
  hipEvent_t end = nullptr;
};

// Launch of a kernel that may be timed: the events are recorded on the launch
// stream just before and just after it.
template <typename F, typename... Args>
inline void launch_maybe_timed(F kernel, dim3 grid, dim3 block, hipStream_t st, TimedLaunch tl, Args... args) {
  if (tl.begin) (void)hipEventRecord(tl.begin, st);
  hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  if (tl.end) (void)hipEventRecord(tl.end, st);
}

// Launchers (defined in the .hip files).  Each returns hipSuccess or the
// launch error.
hipError_t launch_prepare_params(const float* pi, const float* s, uint16_t* derived,
                                 hipStream_t stream);
hipError_t launch_encode_keys(const EncodeArgs& a, int in_bf16, int mse_bits, int qjl, int half,
                              hipStream_t stream, TimedLaunch t);
// Few-token keys (QJL, 2 or 3 index bits) and MSE values (2 or 3 bits) of one
// call in a single launch; hipErrorNotSupported for any other layout or for a
// call the bulk kernels take.
hipError_t launch_encode_small_kv(const EncodeArgs& a, int in_bf16, int key_mse_bits, int key_qjl, int key_half,
                                  int value_bits, hipStream_t stream);
hipError_t launch_encode_values_mse(const EncodeArgs& a, int in_bf16, int bits,
                                    hipStream_t stream, TimedLaunch t);
hipError_t launch_encode_values_minmax(const EncodeArgs& a, int in_bf16, int bits,
                                       hipStream_t stream, TimedLaunch t);
hipError_t launch_ring_append(const void* k_new, const void* v_new, int in_bf16, int batch,
                              int h_kv, uint16_t* ring_k, uint16_t* ring_v, int ring_cap,
                              const SeqValues& n_ring, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int key_mse_bits, int key_qjl, int value_mse,
                         int value_bits, hipStream_t stream, TimedLaunch scan);
// MFMA decode (tq_decode_mfma.hip).  Returns hipErrorNotSupported, having
// launched nothing, for layouts it does not cover.
hipError_t launch_decode_mfma(const DecodeArgs& a, int key_mse_bits, int key_qjl, int value_mse,
                              int value_bits, int key_planes, int value_planes, hipStream_t stream,
                              TimedLaunch scan);
// Workspace bytes of the MFMA path's query digits and constants.
size_t mfma_workspace_bytes(int batch, int h_q, int group);
// The combine step shared by both decode paths.
hipError_t launch_combine(const DecodeArgs& a, int value_mse, hipStream_t stream);

// Device address and size of the static decode scratch on the current device
// (tq_noalloc.hip); the address is looked up on the first call per device.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Work-groups a decode launch aims at (three per compute unit); no slot is
// ever split into more than this many parts.
constexpr int64_t kSplitTarget = 768;
// Decode work split used for the workspace size and the launch.
void decode_split(int64_t max_tokens, int64_t units, int32_t* splits, int32_t* split_len);
// Upper bound of decode_split's split count over all token counts <= max_tokens.
int32_t decode_max_splits(int64_t max_tokens, int64_t units);

}  // namespace tq
