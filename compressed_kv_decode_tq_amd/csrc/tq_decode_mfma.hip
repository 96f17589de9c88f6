// Decode on the matrix cores of gfx950: the compressed scan as MFMAs over the
// stored bit planes.
//
// What is computed (page "03. Results & Benchmarks", "Latency Benchmarks":
// scores, QJL correction, online softmax and value accumulation in one pass;
// page "TurboQuant — Random rotation trước khi quantize, 3-bit KV cache không
// mất accuracy", "Tại sao nó hoạt động": the query is rotated once per step and
// keys are never reconstructed) is the same as the generic scan; only the
// arithmetic is reorganised:
//
// * A symmetric b-bit codebook is affine in the bit planes of the index:
//   c[idx] = cst + sum_p w_p plane_p(idx) (planes bit0..bit2 and bit0^bit1^bit2),
//   so <q_rot, c[idx]> = cst sum(q_rot) + sum_p w_p <q_rot, plane_p>, and the
//   QJL term is <q_s, 2 bit - 1> = 2 <q_s, bit> - sum(q_s).  Every score term is
//   a 0/1-vector times a query vector.
// * Those products run as v_mfma_scale_f32_16x16x128_f8f6f4: the B operand is
//   the bit plane itself as fp4 numbers (a 32-bit plane word becomes the 32
//   nibbles of one lane with one AND per dword, each nibble 0 or a power of
//   two), the A operand the query as four fp8 digits of a float expansion (one
//   digit per MFMA row), whose per-row scales undo the digits' exponents.  One
//   MFMA covers all 128 coordinates of a plane; sums are fp32, and the four
//   digits keep about 16 significant bits of every query coordinate.
// * The value sum sum_t p_t v~_t runs as v_mfma_i32_16x16x64_i8 with the roles
//   swapped: the weights p_t delta_t (min/max) or p_t |v_t| (MSE values) in
//   fixed-point digits, times the value bit planes (bytes holding 2^s, from
//   one AND against 0x01010101 << s; a byte holding 2^7 reads as -128, so the
//   matching digits are negated).  Integer sums are exact.  The score MFMA
//   leaves each lane holding exactly the 16 tokens its digit row needs for the
//   value MFMA, so no data moves between the two.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr float kQjlScale = 0.0097916519f;  // sqrt(pi/2) / 128
constexpr int kScanThreads = 256;           // 4 waves, each scanning its own 64-token chunks

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b),
                                               c, 0, 0, 0);
}

// Bytes of a plane word: byte j of the result is bit (8j + s) of w, scaled by 2^s
// (operand bytes of the MSE-value MFMAs).
__device__ __forceinline__ uint32_t plane_bytes(uint32_t w, int s) { return w & (0x01010101u << s); }

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Score MFMA: A = fp8 (e4m3) query digits, B = fp4 (e2m1) key bits, 16x16x128,
// fp32 accumulation.  sa: the scale of this lane's A row (E8M0, byte 0); B is
// unscaled.
__device__ __forceinline__ floatx4 mfma_f8f4(const i32x8& a, const i32x8& b, floatx4 c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, 0x7F7F7F7F);
}

// fp4 operand of one 32-bit key plane word: nibble j of dword v' holds bit
// 4j + v' of the word as an e2m1 number.  Bits 0, 1 and 2 stay in place (0.5,
// 1, 2: one AND per dword).  Bit 3 of a nibble is e2m1's sign, so dword 3
// keeps it there and sets bit 0 (one AND-OR): the nibble reads +0.5 for a clear
// bit and -0.5 for a set one, i.e. 0.5 - bit.  The query digits carry the
// inverse weights 2, 1, 1/2 and -1; the -1 digits' constant offset
// -0.5 sum(x) over the coordinates of dword 3 (those = 3 mod 4) is taken back
// in the per-head constants.
// k88, k11: 0x88888888 and 0x11111111 held in registers (fp4_masks), so the
// AND-OR is one three-operand instruction rather than two with literals.
__device__ __forceinline__ i32x8 fp4_bits(uint32_t w, uint32_t k88, uint32_t k11) {
  return i32x8{(int)(w & 0x11111111u), (int)(w & 0x22222222u), (int)(w & 0x44444444u),
               (int)((w & k88) | k11), 0, 0, 0, 0};
}
__device__ __forceinline__ void fp4_masks(uint32_t& k88, uint32_t& k11) {
  k88 = 0x88888888u;
  k11 = 0x11111111u;
  asm("" : "+s"(k88), "+v"(k11));  // no instruction: only hides the constants from folding
}

// Coordinate (within the head), log2 of the magnitude of the inverse nibble
// weight, and its sign, of the A element at lane group g, dword v, byte b of
// the score MFMA: the MFMA pairs that element with nibble j' = 4 (v % 2) + b of
// dword v' = 2 (g % 2) + (v / 2) % 2 of lane group g' = 2 (v / 4) + g / 2 of the
// B operand, which holds coordinate 32 g' + 4 j' + v' (so v' = coordinate mod 4).
__device__ __forceinline__ int score_coordinate(int g, int v, int b, int& wexp, bool& neg) {
  const int gp = 2 * (v >> 2) + (g >> 1), vp = 2 * (g & 1) + ((v >> 1) & 1), jp = 4 * (v & 1) + b;
  wexp = vp == 0 ? 1 : (vp == 1 ? 0 : (vp == 2 ? -1 : 0));
  neg = vp == 3;
  return 32 * gp + 4 * jp + vp;
}

// Sum over the 4 lanes of a quad (xor 1, then xor 2) with DPP.
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
  return x;
}

// Max / sum over the 16 lanes of a DPP row (every lane gets the result).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm 1,0,3,2
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm 2,3,0,1
  x = fmaxf(x, dpp<0x124>(x));  // row_ror 4
  return fmaxf(x, dpp<0x128>(x));  // row_ror 8
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x124>(x);
  return x + dpp<0x128>(x);
}

// Max of a non-negative integer over the wave, returned in a scalar register:
// DPP within each 16-lane row, then the four row results through readlane.
__device__ __forceinline__ uint32_t wave_max_u32_uniform(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, true));
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Sum over the four 16-lane rows (every lane gets the sum of its column)
// through the cross-row lane swaps.
__device__ __forceinline__ float col_sum4(float x) {
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(u[0]) + __uint_as_float(u[1]);
}


// Query digits of the score MFMAs.  For head tile ht, score plane pl and A
// lane (g, m), m = 4 hh + L: 32 fp8 bytes, byte b of dword v holding digit L of
// the value x of head 4 ht + hh at the coordinate that element meets in the
// MFMA (score_coordinate), times 2^sigma / (nibble weight).  The index
// planes multiply w_pl * (Pi q) (the shared half/parity word of 3.5-bit keys
// takes w_2 against its low and w_3 against its high 16 bits); the QJL plane,
// the last, 2 * (S q).  The four digits are a
// float expansion: d0 = fp8(y), d1 = fp8(16 (y - d0)), ... (each rounded to
// nearest), so y = d0 + d1/16 + d2/256 + d3/4096 to about 2^-16 relative; the
// MFMA's row scale 2^(-sigma - 4L) undoes the scaling, so the four digit rows
// of a head sum to sum_c x_c bit_c - 0.5 sum_{c = 3 mod 4} x_c (the offset of
// fp4_bits' dword 3, added back through the head constants).  The two products are independent down to
// their digits: work-group (b h, 0) makes the index planes from Pi q (and
// appends the ring token), (b h, 1) the QJL plane from S q.
// One work item is (plane, lane group, head of the tile, dword) of head tile
// ht: it expands the four coordinates of that dword once and writes the dword
// of each of the four digit rows.  x_at(pl, hh, k) is the value plane pl
// multiplies at coordinate k for head 4 ht + hh, s_at(pl, hh) its exponent sigma.
template <class XAt, class SAt>
__device__ __forceinline__ void emit_digits(int tid, int nthreads, int pl0, int pl1, int npl, int ht, int G,
                                            XAt x_at, SAt s_at, uint32_t* dig) {
  const int np = pl1 - pl0;
  const int items = np * 4 * 4 * 8;
  for (int it = tid; it < items; it += nthreads) {
    const int v = it & 7, hh = (it >> 3) & 3, g = (it >> 5) & 3;
    const int pl = pl0 + (it >> 7);
    const int gq = 4 * ht + hh;
    uint32_t word[4] = {0u, 0u, 0u, 0u};
    if (gq < G) {
      const int sg = s_at(pl, hh);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        int wexp;
        bool neg;
        const int k = score_coordinate(g, v, b, wexp, neg);
        const float xk = x_at(pl, hh, k);
        float y = ldexpf(neg ? -xk : xk, sg + wexp);  // |y| < 2^8, inside fp8's range
#pragma unroll
        for (int L = 0; L < 4; ++L) {
          const uint32_t d = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xffu;
          word[L] |= d << (8 * b);
          y = (y - __builtin_amdgcn_cvt_f32_fp8((int)d, 0)) * 16.f;  // exact remainder, next digit
        }
      }
    }
#pragma unroll
    for (int L = 0; L < 4; ++L) dig[(((ht * npl + pl) * 64 + 16 * g + 4 * hh + L) << 3) + v] = word[L];
  }
}

// Per-head digit exponent sigma and score constants of one product (part 0:
// Pi q, part 1: S q) of one head, on one wave.
__device__ __forceinline__ int head_constants(const DecodeArgs& a, const float* x, int part, int lane, int pm,
                                              bool qjl, float* cst) {
  // sr: sum over the coordinates of the base table; srh over the half-bit
  // coordinates (i mod 32 < 16) of the fractional layout; for the QJL part,
  // sr is sum(q_s).  s3, s3h: the same sums over the coordinates = 3 mod 4
  // only (the nibbles that carry 0.5 - bit).
  float mx = 0.f, sr = 0.f, srh = 0.f, s3 = 0.f, s3h = 0.f;
  for (int c = lane; c < kD; c += 64) {
    const float v = x[c];
    const float v3 = (c & 3) == 3 ? v : 0.f;
    mx = fmaxf(mx, fabsf(v));
    if (part == 0 && a.key_half && (c & 31) < 16) {
      srh += v;
      s3h += v3;
    } else {
      sr += v;
      s3 += v3;
    }
  }
  mx = wave_max(mx);
  sr = wave_sum(sr);
  srh = wave_sum(srh);
  s3 = wave_sum(s3);
  s3h = wave_sum(s3h);
  int ex;
  if (part == 0) {
    float wmax = 0.f;
    for (int p = 0; p < pm; ++p) wmax = fmaxf(wmax, fmaxf(fabsf(a.key_w[p]), fabsf(a.key_w_hi[p])));
    frexpf(mx * wmax, &ex);  // |w_p q_rot| < 2^ex
  } else {
    frexpf(2.f * mx, &ex);
  }
  // sigma: the scaled values |x| 2^sigma stay below 2^7 (2^8 after the inverse
  // nibble weight), inside fp8's range of 448; clipped so the row scales
  // 127 - sigma - 4L stay valid E8M0 exponents
  int e = 7 - ex;
  e = e < -100 ? -100 : (e > 100 ? 100 : e);
  if (lane == 0 && cst) {
    if (part == 0) {
      // constant part of <q_rot, c[idx]>, plus the dword-3 offsets of the PM
      // planes: 0.5 sum_p sum_{c = 3 mod 4} w_p(c) q_rot(c)
      float w = 0.f, wh = 0.f;
      for (int p = 0; p < pm; ++p) {
        w += a.key_w[p];
        wh += a.key_w_hi[p];
      }
      cst[0] = a.key_cst * sr + a.key_cst_hi * srh + 0.5f * (s3 * w + (a.key_half ? s3h * wh : 0.f));
      cst[1] = (float)e;                     // sigma of the MSE planes
      if (!qjl) cst[2] = cst[3] = 0.f;  // no QJL plane
    } else {
      cst[2] = (float)e;  // sigma of the QJL plane
      // sum(q_s), less the dword-3 offset of the QJL plane (whose x is 2 q_s):
      // the scan adds -cst[3]
      cst[3] = sr - s3;
    }
  }
  return e;
}

// The step's ring token of slot (b, h), rounded to bf16 (256 threads: the
// first 128 take the key row, the others the value row): ring_token_load reads
// this thread's element (as stored: bf16 or fp32 bits) and its ring position,
// ring_token_store writes it to the ring, so the reads can be issued with the
// work-group's other loads and the write left to the end.
struct RingToken {
  uint32_t raw;
  uint16_t* dst;  // its ring element
};
__device__ __forceinline__ RingToken ring_token_load(const DecodeArgs& a, int b, int h, int tid) {
  // which row is uniform over a wave (128 threads per row): the pointer choice
  // stays in scalar registers
  const int c = tid & (kD - 1), which = __builtin_amdgcn_readfirstlane(tid >> 7);
  const size_t src = ((size_t)b * a.h_kv + h) * kD + c;
  const void* in = which ? a.app_v : a.app_k;
  RingToken r;
  r.raw = a.app_bf16 ? (uint32_t)reinterpret_cast<const uint16_t*>(in)[src]
                     : reinterpret_cast<const uint32_t*>(in)[src];
  r.dst = (which ? a.app_ring_v : a.app_ring_k) + (((size_t)b * a.ring_cap + a.n_ring.v[b] - 1) * a.h_kv + h) * kD + c;
  return r;
}
__device__ __forceinline__ void ring_token_store(const DecodeArgs& a, const RingToken& r) {
  *r.dst = a.app_bf16 ? (uint16_t)r.raw : (uint16_t)f2bf(__uint_as_float(r.raw));
}

template <int MAXG>
struct QueryStage {
  uint32_t raw[MAXG * kD / 256];  // as stored: bf16 or fp32 bits
};
// Queries of virtual heads hoff .. hoff + MAXG - 1 of the slot, on 256
// threads: query_load reads them (every load issued before any is used),
// query_store puts them into LDS, coordinate-major: qt[j][gq/4][gq%4] for head
// hoff + gq.
template <int MAXG>
__device__ __forceinline__ QueryStage<MAXG> query_load(const DecodeArgs& a, int b, int h, int hoff, int tid) {
  QueryStage<MAXG> r;
#pragma unroll
  for (int u = 0; u < MAXG * kD / 256; ++u) {
    const int i = tid + 256 * u, gq = i / kD, c = i % kD;
    int t, hq;
    virtual_head(a, h, hoff + gq < a.group ? hoff + gq : 0, t, hq);
    const size_t off = q_row(a, b, t, hq) * kD + c;
    r.raw[u] = a.q_bf16 ? (uint32_t)reinterpret_cast<const uint16_t*>(a.q)[off]
                        : reinterpret_cast<const uint32_t*>(a.q)[off];
  }
  return r;
}
template <int MAXG>
__device__ __forceinline__ void query_store(const DecodeArgs& a, const QueryStage<MAXG>& r, int hoff, int tid,
                                            floatx4 (*qt)[MAXG / 4]) {
#pragma unroll
  for (int u = 0; u < MAXG * kD / 256; ++u) {
    const int i = tid + 256 * u, gq = i / kD, c = i % kD;
    const float x = a.q_bf16 ? bf2f(r.raw[u]) : __uint_as_float(r.raw[u]);
    reinterpret_cast<float*>(&qt[c][gq >> 2])[gq & 3] = hoff + gq < a.group ? x : 0.f;
  }
}

// Row i of the product's matrix (Pi for part 0, S for part 1), columns
// [j0, j0 + NJ), read from the transposed copies (Pi^T, S^T) so that the
// threads of a wave, which take consecutive rows, read consecutive words: one
// batch of coalesced loads.
template <int NJ>
__device__ __forceinline__ void load_row(const DecodeArgs& a, int part, int i, int j0, float (&m)[NJ]) {
  const float* col = a.mat_t + ((size_t)part * kD + j0) * kD + i;  // M^T[j][i] = M[i][j]
#pragma unroll
  for (int u = 0; u < NJ; ++u) m[u] = col[(size_t)u * kD];
}

// Coordinate i of the product for the MAXG heads from that row and the staged
// queries.
template <int MAXG, int NJ>
__device__ __forceinline__ void row_times_queries(const float (&m)[NJ], int j0, const floatx4 (*qt)[MAXG / 4],
                                                  float (&acc)[MAXG]) {
#pragma unroll
  for (int gq = 0; gq < MAXG; ++gq) acc[gq] = 0.f;
#pragma unroll
  for (int u = 0; u < NJ; ++u)
#pragma unroll
    for (int v = 0; v < MAXG / 4; ++v) {
      const floatx4 qj = qt[j0 + u][v];
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[4 * v + f] = fmaf(m[u], qj[f], acc[4 * v + f]);
    }
}

// LDS of one q-prep part (256 threads).
template <int MAXG>
struct QprepLds {
  floatx4 qt[kD][MAXG / 4];  // queries, coordinate-major
  float qx[MAXG][kD];   // this part's product (Pi q or S q)
  float red[MAXG][kD];  // upper-half partial sums of the product
  int e_head[MAXG];
};

// One q-prep part of head tile ht (heads 4 ht .. 4 ht + 3) of slot (b, h) on
// 256 threads: part 0 makes the index-plane digits from Pi q (and, for tile 0,
// appends the ring token), part 1 the QJL digits from S q.  Thread (hj, i)
// forms coordinate i over the half hj of the columns.  Digits go to dig (the
// slot's nht * npl * 2 * 64 * 4 dwords), per-head constants to cst_base
// ([group][4]).
template <int MAXG>
__device__ __forceinline__ void qprep_part(const DecodeArgs& a, int b, int h, int part, int ht, int tid,
                                           QprepLds<MAXG>& L, uint32_t* dig, float* cst_base, int pm, int pmd,
                                           int npl) {
  static_assert(MAXG == 4, "one head tile per work-group");
  const int G = a.group, hoff = 4 * ht;
  // Loads first, in the order they are needed (ring token, queries, matrix
  // row), so each wait covers only what its use needs; the ring write and the
  // per-head constants' and digits' writes come after the last barrier.
  const bool append = part == 0 && ht == 0 && a.app_k && a.vbase == 0;
  const RingToken rtok = append ? ring_token_load(a, b, h, tid) : RingToken{0u, nullptr};
  const QueryStage<MAXG> qs = query_load<MAXG>(a, b, h, hoff, tid);
  const int i = tid & (kD - 1), hj = tid >> 7;
  float m[kD / 2];
  load_row<kD / 2>(a, part, i, hj * (kD / 2), m);  // in flight while the queries are staged
  query_store<MAXG>(a, qs, hoff, tid, L.qt);
  __syncthreads();
  {
    float acc[MAXG];
    row_times_queries<MAXG, kD / 2>(m, hj * (kD / 2), L.qt, acc);
#pragma unroll
    for (int gq = 0; gq < MAXG; ++gq) (hj ? L.red : L.qx)[gq][i] = acc[gq];
  }
  __syncthreads();
  for (int j = tid; j < MAXG * kD; j += 256) L.qx[j / kD][j % kD] += L.red[j / kD][j % kD];
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6;
  for (int gq = wv; gq < MAXG; gq += 4) {
    const int e = head_constants(a, L.qx[gq], part, lane, pm, npl > pmd,
                                 hoff + gq < G ? cst_base + (hoff + gq) * 4 : nullptr);
    if (lane == 0) L.e_head[gq] = e;
  }
  __syncthreads();
  const int pl0 = part == 0 ? 0 : pmd, pl1 = part == 0 ? pmd : pmd + 1;
  emit_digits(
      tid, 256, pl0, pl1, npl, ht, G,
      [&](int pl, int hh, int k) {
        if (part != 0) return 2.f * L.qx[hh][k];
        // shared word (pmd < pm): bits 0..15 of lane group g's word are the half
        // plane of coordinates 32g..32g+15, bits 16..31 the parity plane of the
        // same coordinates
        if (pmd < pm && pl == 2)
          return (k & 31) < 16 ? a.key_w_hi[2] * L.qx[hh][k] : a.key_w_hi[3] * L.qx[hh][k - 16];
        return (a.key_half && (k & 31) < 16 ? a.key_w_hi[pl] : a.key_w[pl]) * L.qx[hh][k];
      },
      [&](int, int hh) { return L.e_head[hh]; }, dig);
  if (append) ring_token_store(a, rtok);
}

// Separate q-prep kernel of the split scan: work-group (b h, part, head tile).
__global__ __launch_bounds__(256) void qprep_mfma_kernel(DecodeArgs a, int pm, int pmd, int npl, int nht) {
  __shared__ QprepLds<4> lds;
  const int b = __builtin_amdgcn_workgroup_id_x() / a.h_kv, h = __builtin_amdgcn_workgroup_id_x() % a.h_kv;
  uint32_t* dig = reinterpret_cast<uint32_t*>(a.qdig) + (size_t)(b * a.h_kv + h) * (nht * npl * 2 * 64 * 4);
  qprep_part<4>(a, b, h, (int)__builtin_amdgcn_workgroup_id_y(), (int)__builtin_amdgcn_workgroup_id_z(),
                (int)__builtin_amdgcn_workitem_id_x(), lds, dig, a.qconst + ws_row(a, b, h, 0) * 4, pm, pmd, npl);
}

template <int PM, bool QJL, bool VMSE, int PVB, int NHT, bool HALF = false>
__global__ __launch_bounds__(kScanThreads) void scan_mfma_kernel(DecodeArgs a) {
  constexpr int NW = 4;            // waves of the work-group
  constexpr int kRound = 64 * NW;  // tokens the waves take per round of chunks
  constexpr int KB = PM == 1 ? 1 : (PM == 2 ? 2 : 3);  // stored key index planes
  constexpr int KP = KB + (QJL ? 1 : 0);               // stored key planes
  // HALF: index plane KB - 1 is the half plane (16-bit chunk per lane group)
  static_assert(!HALF || (QJL && KB >= 2), "the half-bit layout has QJL and a full plane below the half plane");
  // Half-bit keys with a 3-bit table: Walsh planes 2 (the half plane) and 3
  // (the parity plane) weigh only the half-bit coordinates, so one operand word
  // carries both (the half plane in bits 0..15, the parity of the same
  // coordinates in bits 16..31) and one MFMA scores them.
  constexpr bool SHARED = HALF && PM == 4;
  constexpr int PMD = SHARED ? 3 : PM;                 // index-plane MFMAs
  constexpr int NPL = PMD + (QJL ? 1 : 0);             // score planes
  constexpr int VB = VMSE ? (PVB == 1 ? 1 : (PVB == 2 ? 2 : 3)) : PVB;  // stored value planes
  constexpr int NG = 4;                                // min/max groups of 32 channels
  constexpr int NHEAD = 4 * NHT;

  // per-wave staging of the current chunk, reused at the end for the merge
  // min/max staging is padded so the value-phase reads hit distinct banks:
  // 4 dwords after every 16 tokens of metadata, 16 after every 128 value words
  constexpr int kMetaPad = VMSE ? 0 : 4, kVwPad = VMSE ? 0 : 16;
  constexpr int kStageMeta = 64 * NG + 4 * kMetaPad;  // dwords
  constexpr int kStageNg = 64 * 4;              // floats: per token u = tau log2e n, w = u kappa gamma, mask
  constexpr int kStageVw = 2 * VB * kD + 2 * VB * kVwPad;  // dwords
  constexpr int kStageP = NHEAD * 64;           // floats: p of (head, token) for the value MFMA
  constexpr int kStageTr = VMSE ? 64 * 4 : 64 * 16;  // dwords: value-weight digit blocks, exchanged between lanes
  constexpr int kStage = kStageMeta + kStageNg + kStageVw + kStageP + kStageTr;
  constexpr int kMerge = NHEAD * (kD + 2);
  constexpr int kStride = kStage > kMerge ? kStage : kMerge;
  __shared__ __attribute__((aligned(16))) uint32_t smem[NW * kStride];

  // the wave index is uniform: reading it from the first lane keeps the chunk
  // loop, its bounds and the full/partial chunk test in scalar registers
  const int lane = __builtin_amdgcn_workitem_id_x() & 63, wave = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_workitem_id_x() >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int sh = __builtin_amdgcn_workgroup_id_y();
  const int b = sh / a.h_kv, h = sh % a.h_kv;
  const int G = a.group;
  const int64_t n_c = a.n_comp.v[b];
  const int64_t t_begin = (int64_t)__builtin_amdgcn_workgroup_id_x() * a.split_len;
  const int64_t t_end = t_begin + a.split_len < n_c ? t_begin + a.split_len : n_c;

  uint32_t* s_meta = smem + wave * kStride;
  float* s_ng = reinterpret_cast<float*>(s_meta + kStageMeta);
  uint32_t* s_vw = s_meta + kStageMeta + kStageNg;
  float* s_p = reinterpret_cast<float*>(s_vw + kStageVw);
  uint32_t* s_tr = s_vw + kStageVw + kStageP;

  // query digit operands and per-head constants.  A rows: lane (g, n) supplies
  // row n = (head 4ht + n/4, digit n%4) of the score MFMAs, with the row scale
  // 2^(-sigma - 4 (n%4)) of that head and product; outputs: lane (g, n) holds
  // head 4ht + g's four digit rows for token 16ct + n.
  const u32x4* dig_src = reinterpret_cast<const u32x4*>(a.qdig) + (size_t)sh * NHT * NPL * 64 * 2;
  const float* cst_src = a.qconst + ws_row(a, b, h, 0) * 4;
  i32x8 qa[NHT][NPL];
  {
    const u32x4* src = dig_src;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) {
        const u32x4 lo = src[((ht * NPL + pl) * 64 + lane) * 2], hi = src[((ht * NPL + pl) * 64 + lane) * 2 + 1];
        qa[ht][pl] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
  }
  int sc_m[NHT], sc_s[NHT];  // E8M0 row scales of the index planes and of the QJL plane
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int hq = 4 * ht + (n >> 2);
    const floatx4 cs = hq < G ? *reinterpret_cast<const floatx4*>(cst_src + hq * 4) : floatx4{0.f, 0.f, 0.f, 0.f};
    sc_m[ht] = 0x7F7F7F00 | (127 - (int)cs[1] - 4 * (n & 3));
    sc_s[ht] = 0x7F7F7F00 | (127 - (int)cs[2] - 4 * (n & 3));
  }
  // score of (head, token) in log2 units: u (Sm + c0) + w (Ss - c3), where
  // u = tau log2(e) n, w = u kappa gamma and Sm, Ss are the digit rows' sums;
  // lane (g, n) scores head 4ht + g
  float c0[NHT], c3[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int hq = 4 * ht + g;
    if (hq < G) {
      const floatx4 cs = *reinterpret_cast<const floatx4*>(cst_src + hq * 4);
      c0[ht] = cs[0];
      c3[ht] = cs[3];
    } else {
      c0[ht] = c3[ht] = 0.f;
    }
  }
  const float u_scale = a.scale * 1.4426950409f;  // exp(x) = exp2(x log2 e)
  uint32_t k88, k11;
  fp4_masks(k88, k11);
  // Several causal queries per sequence: the compressed tokens each head of
  // this lane sees (lim) and the fewest any head of the launch sees (lim_min,
  // wave-uniform); chunks that end at or below lim_min need no per-head mask.
  int64_t lim[NHT];
  const int nr_b = (int)a.n_ring.v[b];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    int t, hq, hide_c, hide_r;
    virtual_head(a, h, 4 * ht + g < G ? 4 * ht + g : 0, t, hq);
    hidden_keys(a, t, nr_b, hide_c, hide_r);
    lim[ht] = n_c - hide_c;
  }
  int64_t lim_min;
  {
    int hide_c, hide_r;
    hidden_keys(a, a.vbase / a.qgroup, nr_b, hide_c, hide_r);
    lim_min = n_c - hide_c;
  }

  // key record: full planes of 16 bytes; with HALF the last index plane has 8.
  // The slot's key planes are stored in blocks of 64 tokens (key_word_offset):
  // a chunk is one block, each of its planes one contiguous region.
  const size_t rec = (size_t)KP * (kD / 8) - (HALF ? kD / 16 : 0);
  const uint8_t* kp = a.k_planes + (size_t)sh * key_slot_tokens(a.capacity) * rec;
  const size_t sidx0 = (size_t)sh * a.capacity;
  const uint32_t* vp = a.v_planes + (size_t)sh * (a.capacity >> 5) * VB * kD;

  // Running max m_run (log2 units; starts at a finite floor so exp2(-inf - m)
  // is 0, never NaN) and the reference m_ref of the running sums l_part and
  // acc, which hold sum_t 2^(s_t - m_ref) (...).  p is formed against m_run
  // (so p <= 1 for the value digits) and added with the factor
  // 2^(m_run - m_ref) >= 1; the sums are rescaled to a new reference only when
  // m_run has moved more than kLazyRescale above m_ref (fp32 has the range),
  // so a chunk normally adds to the sums with one fused multiply-add each.
  constexpr float kLazyRescale = 32.f;
  float m_run[NHT], m_ref[NHT], l_part[NHT], acc[NHT][8];
  // sum_t p_t min_t (min/max values) or sum_t p_t |v_t| (MSE values) against
  // m_ref, kept in the weight layout (lane (g, n): head 4ht + n/4 and its own
  // share of the tokens, of group n%4 for min/max values) and added to the
  // channel sums once, after the last chunk
  float macc[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    m_run[ht] = m_ref[ht] = -1e30f;
    l_part[ht] = 0.f;
    macc[ht] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[ht][nt] = 0.f;
  }

  // Chunk loads are issued one chunk ahead: the registers below hold chunk
  // c0t + kRound of this wave while chunk c0t is being computed.  Scalars
  // are kept as loaded (fp16 or fp32 bits) and converted when staged, so no
  // load has to complete before the chunk that uses it.
  uint32_t pX[4][KP];       // key plane words: token 16ct + n, plane word g
  uint32_t pNrm = 0u, pGam = 0u;
  u32x4 pMeta = u32x4{0u, 0u, 0u, 0u};
  u32x4 pVw[VB];
  const int64_t first = t_begin + 64 * wave;
  const int ssz = a.scalar_f16 ? 2 : 4;
  // Addresses are a wave-uniform chunk base (scalar registers) plus a 32-bit
  // per-lane byte offset, so the loads take the scalar-base form and no
  // 64-bit per-lane pointers stay live across the loop.
  // Region of stored plane sp in a key block: 64 times the plane's offset in
  // the record (full planes at 16 sp, the half plane at 16 (KB - 1), the QJL
  // plane after it); lane (g, n) reads words 4 (4n + g) .. + 3 of it, its
  // four column tiles' word g (16-bit words in the half plane).
  auto key_region = [&](int sp) -> int { return 64 * ((HALF && sp == KP - 1) ? sp * (kD / 8) - kD / 16 : sp * (kD / 8)); };
  const uint32_t k_lane = (4 * n + g) * 16u, k_lane_half = (4 * n + g) * 8u;
  const uint32_t s_lane = lane * (uint32_t)ssz;       // token `lane`'s scalar
  const uint32_t m_lane = VMSE ? s_lane : lane * (uint32_t)(NG * 4);
  const uint32_t v_lane = lane * 16u;                 // four value words per lane
  // The compressed cache is read once per step: its loads are non-temporal
  // (streamed past the caches instead of displacing the query digits and the
  // per-head constants every work-group reuses).
  auto scalar_bits = [&](const void* base, uint32_t off) -> uint32_t {
    const char* p = reinterpret_cast<const char*>(base) + off;
    return a.scalar_f16 ? (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p))
                        : __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  };
  auto scalar_value = [&](uint32_t bits) -> float {
    return a.scalar_f16 ? __half2float(__ushort_as_half((unsigned short)bits)) : __uint_as_float(bits);
  };
  // The keys of a chunk: a whole 64-token block, read without per-lane guards
  // even for a partial chunk (the block is allocated; tokens past the end get
  // a -inf score from the staged mask, and fp4 bits are always finite).
  auto load_keys = [&](int64_t c) {
    const uint8_t* xk = kp + (c >> 6) * (int64_t)(64 * rec);
#pragma unroll
    for (int sp = 0; sp < KP; ++sp) {
      if (HALF && sp == KB - 1) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(xk + key_region(sp) + k_lane_half));
        pX[0][sp] = v[0] & 0xffffu;
        pX[1][sp] = v[0] >> 16;
        pX[2][sp] = v[1] & 0xffffu;
        pX[3][sp] = v[1] >> 16;
      } else {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xk + key_region(sp) + k_lane));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) pX[ct][sp] = v[ct];
      }
    }
  };
  // The per-token data and value words of a chunk (guarded past its end).
  auto load_rest = [&](int64_t c) {
    const int rem_c = (int)(t_end - c < 64 ? t_end - c : 64);
    const char* xn = reinterpret_cast<const char*>(a.k_norm) + (int64_t)(sidx0 + c) * ssz;
    const char* xg = QJL ? reinterpret_cast<const char*>(a.k_rnorm) + (int64_t)(sidx0 + c) * ssz : nullptr;
    const char* xm = VMSE ? reinterpret_cast<const char*>(a.v_norm) + (int64_t)(sidx0 + c) * ssz
                          : reinterpret_cast<const char*>(a.v_meta) + (int64_t)(sidx0 + c) * (NG * 4);
    const char* xv = reinterpret_cast<const char*>(vp + (c >> 5) * VB * kD);
    if (rem_c == 64) {  // full chunk: no per-lane guards
      pNrm = scalar_bits(xn, s_lane);
      if (QJL) pGam = scalar_bits(xg, s_lane);
      if (VMSE)
        pMeta[0] = scalar_bits(xm, m_lane);
      else
        pMeta = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xm + m_lane));
#pragma unroll
      for (int i = 0; i < VB; ++i) pVw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xv + v_lane + i * 1024));
    } else {
      const bool valid = lane < rem_c;
      pNrm = valid ? scalar_bits(xn, s_lane) : 0u;
      pGam = (QJL && valid) ? scalar_bits(xg, s_lane) : 0u;
      if (VMSE)
        pMeta[0] = valid ? scalar_bits(xm, m_lane) : 0u;
      else
        pMeta = valid ? *reinterpret_cast<const u32x4*>(xm + m_lane) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < VB; ++i) {
        const int idx = (i * 64 + lane) * 4;  // dword index inside [2][VB][128]
        pVw[i] = (idx < VB * kD || rem_c > 32) ? *reinterpret_cast<const u32x4*>(xv + v_lane + i * 1024)
                                               : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  if (first < t_end) {
    load_rest(first);
    load_keys(first);
  }

  for (int64_t c0t = first; c0t < t_end; c0t += kRound) {
    const int rem = (int)(t_end - c0t < 64 ? t_end - c0t : 64);  // valid tokens of this chunk
    // ---- stage this chunk's per-token data and value words in LDS; the
    // value-weight exponent comes from the largest delta (min/max values) or
    // |v| (MSE values) of the chunk, as bits (non-negative: integer order is
    // float order)
    const float vnorm = VMSE ? scalar_value(pMeta[0]) : 0.f;  // |v| (MSE values)
    const uint32_t mb_lane = VMSE ? __float_as_uint(vnorm)
                                  : max(max(pMeta[0] & 0x7fffu, pMeta[1] & 0x7fffu),
                                        max(pMeta[2] & 0x7fffu, pMeta[3] & 0x7fffu));
    // min/max values: the exponent of the value weights is known before the
    // softmax, so p is produced already scaled (see the value section)
    const int ev_mm = VMSE ? 0 : 44 - (int)(wave_max_u32_uniform(mb_lane) >> 10);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    {
      // per token: u, w and an additive mask (-inf past the end of the chunk)
      const float u = u_scale * scalar_value(pNrm);
      *reinterpret_cast<floatx4*>(s_ng + 4 * lane) =
          floatx4{u, QJL ? u * kQjlScale * scalar_value(pGam) : 0.f, lane < rem ? 0.f : -INFINITY, 0.f};
      if (VMSE)
        s_meta[lane * NG] = __float_as_uint(vnorm);
      else
        *reinterpret_cast<u32x4*>(s_meta + lane * NG + kMetaPad * (lane >> 4)) = pMeta;
#pragma unroll
      for (int i = 0; i < VB; ++i) {
        const int q = (i * 64 + lane) * 4;  // word index inside the chunk's value words
        *reinterpret_cast<u32x4*>(s_vw + q + kVwPad * (q >> 7)) = pVw[i];
      }
    }
    uint32_t(&X)[4][KP] = pX;  // the key words are reloaded once the scores are done
    if (c0t + kRound < t_end) load_rest(c0t + kRound);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- scores (log2 units).  The query digits are the A operand and the
    // key bits the B operand (fp4, one MFMA per plane covers all 128
    // coordinates), so lane (g, n) receives, for token 16ct + n and head 4ht + g,
    // all four digit rows (accumulator element r = digit r), already scaled.
    float sc[NHT][4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      uint32_t P[PM];
      P[0] = X[ct][0];
      if (PM >= 2) P[1 % PM] = X[ct][1 % KP];
      if (SHARED) {
        // the half plane's word has its 16 bits at the bottom; the parity of
        // the same coordinates goes above them
        P[2 % PM] = X[ct][2 % KP] | ((X[ct][0] ^ X[ct][1 % KP] ^ X[ct][2 % KP]) << 16);
      } else if (PM == 4) {
        P[2 % PM] = X[ct][2 % KP];
        P[3 % PM] = X[ct][0] ^ X[ct][1 % KP] ^ X[ct][2 % KP];
      }
      // the constants enter through the accumulators (element 0: digit row 0)
      floatx4 cm[NHT], cq[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        cm[ht] = floatx4{c0[ht], 0.f, 0.f, 0.f};
        cq[ht] = floatx4{-c3[ht], 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int pl = 0; pl < PMD; ++pl) {
        const i32x8 Bk = fp4_bits(P[pl], k88, k11);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) cm[ht] = mfma_f8f4(qa[ht][pl], Bk, cm[ht], sc_m[ht]);
      }
      if (QJL) {
        const i32x8 Bk = fp4_bits(X[ct][KP - 1], k88, k11);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) cq[ht] = mfma_f8f4(qa[ht][NPL - 1], Bk, cq[ht], sc_s[ht]);
      }
      const int u = 16 * ct + n;  // token inside the chunk
      const floatx4 ng = *reinterpret_cast<const floatx4*>(s_ng + 4 * u);
      const float ut = ng[0], wt = ng[1];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        float sv = fmaf(ut, (cm[ht][0] + cm[ht][1]) + (cm[ht][2] + cm[ht][3]), ng[2]);
        if (QJL) sv = fmaf(wt, (cq[ht][0] + cq[ht][1]) + (cq[ht][2] + cq[ht][3]), sv);
        sc[ht][ct] = sv;
      }
    }
    if (c0t + 64 > lim_min) {  // tail of the compressed part under a causal query
      // (a wave-uniform branch, kept a branch: the per-lane selects below run
      // only in the chunks that need them)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) sc[ht][ct] = c0t + 16 * ct + n < lim[ht] ? sc[ht][ct] : -INFINITY;
    }

    if (c0t + kRound < t_end) load_keys(c0t + kRound);

    // ---- online softmax in log2 units over the 16 lanes of a head (one DPP
    // row), with the lazily rescaled sums above.  p goes to LDS for the value MFMA,
    // for min/max values as p 2^c with c = ev - 2 min(n/4, 2): token 16ct + n
    // is in slot n/4 of its packed code word, whose bytes carry 4^min(n/4, 2)
    // (4-bit codes: every slot is one whole code per byte, no scale)
    const int c_p = VMSE ? 0 : (VB == 4 ? ev_mm : ev_mm - ((n >> 2) < 2 ? 2 * (n >> 2) : 4));
    float lsum[NHT];
    bool far = false;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const float mloc = row_max16(fmaxf(fmaxf(sc[ht][0], sc[ht][1]), fmaxf(sc[ht][2], sc[ht][3])));
      const float m_new = fmaxf(m_run[ht], mloc);
      m_run[ht] = m_new;
      far |= m_new - m_ref[ht] > kLazyRescale;
      const float m_p = m_new - (float)c_p;
      lsum[ht] = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const float e = __builtin_amdgcn_exp2f(sc[ht][ct] - m_p);  // 0 for tokens past the end
        s_p[(4 * ht + g) * 64 + 16 * ct + n] = e;
        lsum[ht] += e;
      }
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(far) != 0, 0)) {  // wave-uniform: a new reference for every lane
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const float f = __builtin_amdgcn_exp2f(m_ref[ht] - m_run[ht]);
        l_part[ht] *= f;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[ht][nt] *= f;
        {  // macc: the factor of head 4ht + n/4 (DPP row n/4), through scalar registers
          const float f0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 0));
          const float f1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 16));
          const float f2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 32));
          const float f3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 48));
          const int q = n >> 2;
          macc[ht] *= q == 0 ? f0 : (q == 1 ? f1 : (q == 2 ? f2 : f3));
        }
        m_ref[ht] = m_run[ht];
      }
    }
    float beta[NHT];  // 2^(m_run - m_ref) of the accumulator rows: head 4ht + g
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      beta[ht] = __builtin_amdgcn_exp2f(m_run[ht] - m_ref[ht]);
      l_part[ht] = fmaf(VMSE ? lsum[ht] : ldexpf(lsum[ht], -c_p), beta[ht], l_part[ht]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- values
    if (!VMSE) {
      static_assert(VMSE || VB == 2 || VB == 4, "min/max values on this path are 2- or 4-bit packed codes");
      // Rows of the value MFMA are (head 4ht + n/4, group n%4) and this lane
      // supplies tokens 16g + 4k + r (k, r < 4): the tokens of the packed code
      // word g of the chunk, whose AND with 0x03 << 2k (k < 3), or with 0x30
      // after a shift by 2 (k = 3), leaves code(16g + 4k + r) * 4^min(k, 2) in
      // byte r.  The weights p_t delta_t(group) carry the inverse scale and
      // become signed base-256 fixed point.
      const int grp = n & 3;
      // ev = 44 - E(max delta): every delta < 2^(E - 14), so |W| < 2^30.  The
      // weights p delta 2^(ev - 2 min(k, 2)) come straight from the scaled p.
      const float inv_sv = ldexpf(1.f, -ev_mm);
      // one head tile at a time (its digit operands, then its eight channel
      // tiles), so a second tile does not double the live registers
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        floatx4 pv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pv[k] = *reinterpret_cast<const floatx4*>(s_p + (4 * ht + (n >> 2)) * 64 + 16 * g + 4 * k);
        u32x4 A[4];
        float Mk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t V[4];
          Mk[k] = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t mm = s_meta[(16 * g + 4 * k + r) * NG + kMetaPad * g + grp];
            const float dl = __half2float(__ushort_as_half((unsigned short)(mm & 0xffffu)));
            const float mn = __half2float(__ushort_as_half((unsigned short)(mm >> 16)));
            const float pe = pv[k][r];
            const int W = (int)fmaf(pe, dl, 0.5f);  // non-negative: rounds to nearest
            // signed base-256 digits are the bytes of (W + 0x808080) ^ 0x808080;
            // the XOR of the three low bytes is applied after the transpose
            V[r] = (uint32_t)W + 0x00808080u;
            Mk[k] = fmaf(pe, mn, Mk[k]);
          }
          // 4x4 byte transpose: digit plane d holds byte d of the four tokens
          const uint32_t t01lo = __builtin_amdgcn_perm(V[1], V[0], 0x05010400u);
          const uint32_t t01hi = __builtin_amdgcn_perm(V[1], V[0], 0x07030602u);
          const uint32_t t23lo = __builtin_amdgcn_perm(V[3], V[2], 0x05010400u);
          const uint32_t t23hi = __builtin_amdgcn_perm(V[3], V[2], 0x07030602u);
          A[3][k] = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u) ^ 0x80808080u;  // least significant digit
          A[2][k] = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u) ^ 0x80808080u;
          A[1][k] = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u) ^ 0x80808080u;
          A[0][k] = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);  // most significant digit
        }
        // this lane's part of sum_t p_t min_t for (head 4ht + n/4, group n%4),
        // the slot scales 2^(ev - 2 min(k, 2)) undone, added against m_ref with
        // that head's factor 2^(m_run - m_ref) (held by DPP row n/4)
        const float mk = VB == 4 ? (Mk[0] + Mk[1]) + (Mk[2] + Mk[3])
                                 : fmaf(Mk[0], 1.f, fmaf(Mk[1], 4.f, 16.f * (Mk[2] + Mk[3])));
        macc[ht] = fmaf(mk, inv_sv * __shfl(beta[ht], 16 * (n >> 2) + n), macc[ht]);
        // Exchange the digit blocks inside each quad of lanes: lane (g, 4h + G)
        // holds digit d of row (head h, group G) in A[d]; the value MFMA of
        // group G takes rows (head h, digit d) from lane (g, 4h + d), so one
        // MFMA per channel tile yields all four digits of its own group.  Block
        // d of lane L sits at slot d * 64 + (L ^ d): writes and reads both
        // cover all banks once per 16 lanes.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int d = 0; d < 4; ++d) *reinterpret_cast<u32x4*>(s_tr + 4 * (d * 64 + (lane ^ d))) = A[d];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        u32x4 AG[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          AG[gi] = *reinterpret_cast<const u32x4*>(s_tr + 4 * ((n & 3) * 64 + ((lane & ~3) | (gi ^ (n & 3)))));
        auto value_operand = [&](int nt) -> u32x4 {
          if (VB == 4) {
            // 4-bit codes: tokens 16g..16g+15 are the staged rows 2g and 2g+1
            // (eight tokens each); token i of a word sits in byte i%4, nibble i/4
            const uint32_t w0 = s_vw[(2 * g) * (kD + kVwPad) + 16 * nt + n];
            const uint32_t w1 = s_vw[(2 * g + 1) * (kD + kVwPad) + 16 * nt + n];
            return u32x4{w0 & 0x0f0f0f0fu, (w0 >> 4) & 0x0f0f0f0fu, w1 & 0x0f0f0f0fu, (w1 >> 4) & 0x0f0f0f0fu};
          }
          const uint32_t w = s_vw[g * (kD + kVwPad) + 16 * nt + n];
          return u32x4{w & 0x03030303u, w & 0x0c0c0c0cu, w & 0x30303030u, (w >> 2) & 0x30303030u};
        };
        // rows (head g, digit r) of group nt/2 (channels 16nt..16nt+15):
        // element r is digit r's product.  The MFMA of tile nt + 1 is issued
        // before the result of tile nt is read, so its latency overlaps.
        const float s_acc = inv_sv * beta[ht];  // weight scale and reference factor of head 4ht + g
        i32x4 Cn = mfma_i8(AG[0], value_operand(0), i32x4{0, 0, 0, 0});
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const i32x4 C = Cn;
          if (nt + 1 < 8) Cn = mfma_i8(AG[(nt + 1) >> 1], value_operand(nt + 1), i32x4{0, 0, 0, 0});
          const float v = fmaf((float)((C[0] << 8) + C[1]), 65536.f, (float)((C[2] << 8) + C[3]));
          acc[ht][nt] = fmaf(v, s_acc, acc[ht][nt]);
        }
      }
    } else {
      // MSE values: weights W = p_t |v_t| (the same for every value plane),
      // accumulated in rotated space.  Rows of the value MFMA are (head, digit);
      // its K slot (dword c, byte r) holds token 16c + 4g + r, whose value bit
      // sits at bit s = 4 (c % 2) + g of its byte (bit-plane order), so W enters
      // as W 2^(ev - s) and a byte holding 2^7 reads as -128 (W negated there).
      // Lane (g, 4h + c) forms W for head 4ht + h and the four tokens 16c + 4g + r
      // only (no lane repeats another's), as signed base-256 digits; a quad
      // exchange through LDS then gives lane (g, 4h + d) digit d of all sixteen.
      const uint32_t mb = wave_max_u32_uniform(mb_lane);
      int ex;
      frexpf(__uint_as_float(mb), &ex);
      const int ev = 30 - ex;  // |W 2^ev| < 2^30
      const float inv_sv = ldexpf(1.f, -ev);
      const int cq = n & 3, s_tok = 4 * (cq & 1) + g;
      const float sc = s_tok == 7 ? -ldexpf(1.f, ev - 7) : ldexpf(1.f, ev - s_tok);
      const float half = s_tok == 7 ? -0.5f : 0.5f;  // rounds |W| to nearest
      float nvs[4], nvr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        nvr[r] = __uint_as_float(s_meta[(16 * cq + 4 * g + r) * NG]);
        nvs[r] = nvr[r] * sc;
      }
      u32x4 A[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const floatx4 pq = *reinterpret_cast<const floatx4*>(s_p + (4 * ht + (n >> 2)) * 64 + 16 * cq + 4 * g);
        uint32_t V[4];
        float pn = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          V[r] = (uint32_t)(int)fmaf(pq[r], nvs[r], half) + 0x00808080u;
          pn = fmaf(pq[r], nvr[r], pn);
        }
        // this lane's part of sum_t p_t |v_t| for head 4ht + n/4, against m_ref
        macc[ht] = fmaf(pn, __shfl(beta[ht], 16 * (n >> 2) + n), macc[ht]);
        // 4x4 byte transpose: D[d] holds digit d of the four tokens
        uint32_t D[4];
        const uint32_t t01lo = __builtin_amdgcn_perm(V[1], V[0], 0x05010400u);
        const uint32_t t01hi = __builtin_amdgcn_perm(V[1], V[0], 0x07030602u);
        const uint32_t t23lo = __builtin_amdgcn_perm(V[3], V[2], 0x05010400u);
        const uint32_t t23hi = __builtin_amdgcn_perm(V[3], V[2], 0x07030602u);
        D[3] = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u) ^ 0x80808080u;  // least significant digit
        D[2] = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u) ^ 0x80808080u;
        D[1] = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u) ^ 0x80808080u;
        D[0] = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);  // most significant digit
        // quad exchange: digit d of lane L at slot 64 d + (L ^ d); lane (g, 4h + d)
        // reads dword c from lane (g, 4h + c)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int d = 0; d < 4; ++d) s_tr[64 * d + (lane ^ d)] = D[d];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int c = 0; c < 4; ++c) A[ht][c] = s_tr[64 * cq + (((lane & ~3) | c) ^ cq)];
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int ch = 16 * nt + n;
        float vs[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) vs[ht] = 0.f;
        uint32_t Wd[4][VB];
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int pv = 0; pv < VB; ++pv) Wd[d][pv] = s_vw[((d >> 1) * VB + pv) * kD + ch];
        u32x4 Bp[VB];
#pragma unroll
        for (int pl = 0; pl < PVB; ++pl) {
          u32x4 B;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            if (pl < VB) {
              B[d] = plane_bytes(Wd[d][pl % VB], 4 * (d & 1) + g);
              Bp[pl % VB][d] = B[d];
            } else {  // the parity plane: the AND distributes over the XOR
              B[d] = Bp[0][d] ^ Bp[1 % VB][d] ^ Bp[2 % VB][d];
            }
          }
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) {
            const i32x4 C = mfma_i8(A[ht], B, i32x4{0, 0, 0, 0});
            const float v = fmaf((float)((C[0] << 8) + C[1]), 65536.f, (float)((C[2] << 8) + C[3]));
            vs[ht] = fmaf(v, a.val_w[pl], vs[ht]);
          }
        }
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) acc[ht][nt] = fmaf(vs[ht], inv_sv * beta[ht], acc[ht][nt]);
      }
    }
  }

  if (!VMSE) {
    // the min terms: reduce over the four token quarters, then fetch (head g,
    // group gi) into the channel layout
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const float x = col_sum4(macc[ht]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[ht][nt] += __shfl(x, 4 * g + (nt >> 1));
    }
  } else {
    // the constant of the value codebook times sum_t p_t |v_t|: reduce over the
    // sixteen lanes of each head, then fetch head g
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const float x = __shfl(quad_sum(col_sum4(macc[ht])), 4 * g);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[ht][nt] = fmaf(a.val_cst, x, acc[ht][nt]);
    }
  }

  // ---- merge the four waves: one (m, l, acc[128]) partial per query head,
  // with m converted back to natural-log units
  float lsum[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) lsum[ht] = row_sum16(l_part[ht]);  // the 16 lanes of head 4ht + g
  // (the sums are relative to m_ref, which is therefore the partial's max)
  __syncthreads();
  float* mrg = reinterpret_cast<float*>(smem) + wave * kStride;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    if (n == 0) {
      const int hh = 4 * ht + g;
      mrg[hh * (kD + 2)] = lsum[ht] > 0.f ? m_ref[ht] * 0.6931471806f : -INFINITY;
      mrg[hh * (kD + 2) + 1] = lsum[ht];
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) mrg[(4 * ht + g) * (kD + 2) + 2 + 16 * nt + n] = acc[ht][nt];
  }
  __syncthreads();
  const float* base = reinterpret_cast<const float*>(smem);
  for (int i = __builtin_amdgcn_workitem_id_x(); i < G * kD; i += kScanThreads) {
    const int hh = i / kD, c = i % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, base[w * kStride + hh * (kD + 2)]);
    float L = 0.f, Acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = base[w * kStride + hh * (kD + 2)];
        const float f = mw == -INFINITY ? 0.f : __expf(mw - M);
        L += f * base[w * kStride + hh * (kD + 2) + 1];
        Acc += f * base[w * kStride + hh * (kD + 2) + 2 + c];
      }
    }
    float* part = a.partial + ((size_t)__builtin_amdgcn_workgroup_id_x() * a.batch * a.h_kv * G + ws_row(a, b, h, hh)) * (kD + 2);
    if (c == 0) {
      part[0] = M;
      part[1] = L;
    }
    part[2 + c] = Acc;
  }
}

template <int PM, bool QJL, bool VMSE, int PVB, int NHT, bool HALF = false>
hipError_t launch_scan_mfma(const DecodeArgs& a, hipStream_t st, TimedLaunch tl) {
  launch_maybe_timed(scan_mfma_kernel<PM, QJL, VMSE, PVB, NHT, HALF>, dim3(a.splits, a.batch * a.h_kv),
                     dim3(kScanThreads), st, tl, a);
  return hipGetLastError();
}

template <int NHT>
hipError_t dispatch_mfma(const DecodeArgs& a, int kb, int qjl, int vmse, int vb, hipStream_t st,
                         TimedLaunch tl) {
  if (!qjl) {  // keys without the QJL bit (the MSE-only quantizer)
    if (a.key_half) return hipErrorNotSupported;
    if (kb == 1 && !vmse && vb == 2) return launch_scan_mfma<1, false, false, 2, NHT>(a, st, tl);
    if (kb == 1 && !vmse && vb == 4) return launch_scan_mfma<1, false, false, 4, NHT>(a, st, tl);
    if (kb == 1 && vmse && vb == 3) return launch_scan_mfma<1, false, true, 4, NHT>(a, st, tl);
    if (kb == 2 && !vmse && vb == 2) return launch_scan_mfma<2, false, false, 2, NHT>(a, st, tl);
    if (kb == 2 && !vmse && vb == 4) return launch_scan_mfma<2, false, false, 4, NHT>(a, st, tl);
    if (kb == 3 && !vmse && vb == 2) return launch_scan_mfma<4, false, false, 2, NHT>(a, st, tl);
    if (kb == 3 && !vmse && vb == 4) return launch_scan_mfma<4, false, false, 4, NHT>(a, st, tl);
    if (kb == 2 && vmse && vb == 3) return launch_scan_mfma<2, false, true, 4, NHT>(a, st, tl);
    if (kb == 3 && vmse && vb == 3) return launch_scan_mfma<4, false, true, 4, NHT>(a, st, tl);
    return hipErrorNotSupported;
  }
  if (a.key_half) {  // kb counts the half plane: 1 + 1/2 or 2 + 1/2 MSE bits
    if (kb == 2 && !vmse && vb == 2) return launch_scan_mfma<2, true, false, 2, NHT, true>(a, st, tl);
    if (kb == 2 && !vmse && vb == 4) return launch_scan_mfma<2, true, false, 4, NHT, true>(a, st, tl);
    if (kb == 3 && !vmse && vb == 2) return launch_scan_mfma<4, true, false, 2, NHT, true>(a, st, tl);
    if (kb == 3 && !vmse && vb == 4) return launch_scan_mfma<4, true, false, 4, NHT, true>(a, st, tl);
    if (kb == 2 && vmse && vb == 3) return launch_scan_mfma<2, true, true, 4, NHT, true>(a, st, tl);
    if (kb == 3 && vmse && vb == 3) return launch_scan_mfma<4, true, true, 4, NHT, true>(a, st, tl);
    return hipErrorNotSupported;
  }
  if (kb == 1 && !vmse && vb == 2) return launch_scan_mfma<1, true, false, 2, NHT>(a, st, tl);
  if (kb == 1 && !vmse && vb == 4) return launch_scan_mfma<1, true, false, 4, NHT>(a, st, tl);
  if (kb == 1 && vmse && vb == 3) return launch_scan_mfma<1, true, true, 4, NHT>(a, st, tl);
  if (kb == 2 && !vmse && vb == 2) return launch_scan_mfma<2, true, false, 2, NHT>(a, st, tl);
  if (kb == 2 && !vmse && vb == 4) return launch_scan_mfma<2, true, false, 4, NHT>(a, st, tl);
  if (kb == 3 && !vmse && vb == 2) return launch_scan_mfma<4, true, false, 2, NHT>(a, st, tl);
  if (kb == 3 && !vmse && vb == 4) return launch_scan_mfma<4, true, false, 4, NHT>(a, st, tl);
  if (kb == 2 && vmse && vb == 3) return launch_scan_mfma<2, true, true, 4, NHT>(a, st, tl);
  if (kb == 3 && vmse && vb == 3) return launch_scan_mfma<4, true, true, 4, NHT>(a, st, tl);
  if (kb == 2 && vmse && vb == 2) return launch_scan_mfma<2, true, true, 2, NHT>(a, st, tl);
  if (kb == 3 && vmse && vb == 2) return launch_scan_mfma<4, true, true, 2, NHT>(a, st, tl);
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a_in, int key_mse_bits, int key_qjl, int value_mse,
                              int value_bits, int key_planes, int value_planes, hipStream_t stream,
                              TimedLaunch tl) {
  // covered: keys with 1-, 2- or 3-bit indices (or 1.5 / 2.5 with QJL), with
  // or without the QJL bit, 2- or 4-bit min/max values in groups of 32 or
  // 3-bit MSE values (2-bit MSE values with 2+1- and 3+1-bit keys),
  // antisymmetric codebooks, up to 8 query heads per KV head
  if (key_mse_bits < 1 || key_mse_bits > 3) return hipErrorNotSupported;
  if (!key_qjl && a_in.key_half) return hipErrorNotSupported;
  if (key_planes != (1 << (key_mse_bits - 1))) return hipErrorNotSupported;
  if (value_mse) {
    if ((value_bits != 2 && value_bits != 3) || value_planes != (1 << (value_bits - 1))) return hipErrorNotSupported;
    if (value_bits == 2 && (!key_qjl || a_in.key_half || key_mse_bits < 2)) return hipErrorNotSupported;
  } else if ((value_bits != 2 && value_bits != 4) || a_in.value_group != 32) {
    return hipErrorNotSupported;
  }
  if (a_in.group > 8) return hipErrorNotSupported;
  const int nht = a_in.group > 4 ? 2 : 1;
  const DecodeArgs& a = a_in;
  const int pm = 1 << (key_mse_bits - 1);
  // half-bit keys with a 3-bit table: Walsh planes 2 and 3 share one operand
  // word (the scan's SHARED layout), so the index product has three digit planes
  const int pmd = (a.key_half && pm == 4) ? 3 : pm;
  const int npl = pmd + (key_qjl ? 1 : 0);
  const dim3 qgrid(a.batch * a.h_kv, key_qjl ? 2 : 1, nht);
  hipLaunchKernelGGL(qprep_mfma_kernel, qgrid, dim3(256), 0, stream, a, pm, pmd, npl, nht);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = nht == 1 ? dispatch_mfma<1>(a, key_mse_bits, key_qjl, value_mse, value_bits, stream, tl)
               : dispatch_mfma<2>(a, key_mse_bits, key_qjl, value_mse, value_bits, stream, tl);
  if (e != hipSuccess) return e;
  return launch_combine(a, value_mse, stream);
}

}  // namespace tq
