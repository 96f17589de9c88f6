// Decode on the int8 matrix cores of gfx950: the compressed scan as integer
// MFMAs over the stored bit planes.
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
// * Those products run as v_mfma_i32_16x16x64_i8: one operand is the bit plane
//   itself (a byte per bit, taken from a 32-bit plane word with ONE AND against
//   0x01010101 << s, so the byte holds 2^s), the other the query in fixed point
//   split into four signed base-128 digits (one digit per MFMA row/column),
//   pre-scaled by 2^-s to cancel the byte's 2^s.  Integer sums are exact; the
//   fixed point keeps 20+ significant bits of every query coordinate.
// * The value sum sum_t p_t v~_t runs the same way with the roles swapped: the
//   weights p_t delta_t (min/max) or p_t |v_t| (MSE values) in fixed-point
//   digits, times the value bit planes.  The score MFMA leaves each lane holding
//   exactly the 16 tokens its digit row needs for the value MFMA, so no data
//   moves between the two.
// * A byte holding 2^7 reads as -128 in int8; the matching digits are negated.
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

// Bytes of a plane word: byte j of the result is bit (8j + s) of w, scaled by 2^s.
__device__ __forceinline__ uint32_t plane_bytes(uint32_t w, int s) { return w & (0x01010101u << s); }

// Signed base-128 digits of q (|q| < 2^27), most significant first.
__device__ __forceinline__ void digits128(int q, int d[4]) {
#pragma unroll
  for (int L = 3; L >= 1; --L) {
    const int r = ((q + 64) & 127) - 64;
    d[L] = r;
    q = (q - r) >> 7;
  }
  d[0] = q;
}

// Query digits: for head tile ht, score plane pl, contraction half hf and lane
// (g, n), 16 bytes: byte 4d + j holds digit n%4 of head 4ht + n/4 at
// coordinate k = 32g + 8j + 4hf + d, pre-scaled by 2^-(k%8) (negated for
// k%8 == 7).  Plane pl < PM multiplies w_pl * (Pi q); plane PM (QJL) 2 * (S q).
// The two products are independent down to their digits: work-group (b h, 0)
// makes the PM index planes from Pi q (and appends the ring token), (b h, 1)
// the QJL plane from S q.
template <int MAXG>
__global__ __launch_bounds__(256) void qprep_mfma_kernel(DecodeArgs a, int pm, int npl, int nht) {
  constexpr int NQ = MAXG / 4;               // float4 groups of heads per coordinate
  __shared__ floatx4 qt[kD][NQ];             // queries, coordinate-major: qt[j][gq/4][gq%4]
  __shared__ float qx[kMaxGroup][kD];        // this part's product (Pi q or S q)
  __shared__ float red[kMaxGroup][kD];       // upper-half partial sums of the product
  __shared__ int e_head[kMaxGroup];
  const int b = blockIdx.x / a.h_kv, h = blockIdx.x % a.h_kv;
  const int part = blockIdx.y;               // 0: Pi q, index planes; 1: S q, QJL plane
  const int G = a.group;
  if (part == 0 && a.app_k && a.vbase == 0) {
    // fused ring append: threads 0..127 write the key row, 128..255 the value
    // row of this (sequence, KV head), rounded to bf16 as the ring append does
    const int c = threadIdx.x & (kD - 1), which = threadIdx.x >> 7;
    const size_t src = ((size_t)b * a.h_kv + h) * kD + c;
    const size_t dst = (((size_t)b * a.ring_cap + a.n_ring.v[b] - 1) * a.h_kv + h) * kD + c;
    const void* in = which ? a.app_v : a.app_k;
    uint16_t* ring = which ? a.app_ring_v : a.app_ring_k;
    ring[dst] = a.app_bf16 ? reinterpret_cast<const uint16_t*>(in)[src]
                           : (uint16_t)f2bf(reinterpret_cast<const float*>(in)[src]);
  }
  // thread (hj, i): coordinates j of half hj of row i of the product; column
  // j of the matrix is row j of its transpose, so consecutive threads read
  // consecutive words.  The 64 matrix loads go out before the queries are
  // staged, so both round trips overlap.
  const int i_row = threadIdx.x & (kD - 1);
  const int hj = threadIdx.x >> 7;
  float w[kD / 2];
  {
    const float* mt = a.mat_t + (size_t)part * kD * kD + (size_t)(hj * (kD / 2)) * kD + i_row;
#pragma unroll
    for (int j = 0; j < kD / 2; ++j) w[j] = mt[(size_t)j * kD];
  }
  for (int i = threadIdx.x; i < MAXG * kD; i += blockDim.x) {
    const int gq = i / kD, c = i % kD;
    float x = 0.f;
    if (gq < G) {
      int t, hq;
      virtual_head(a, h, gq, t, hq);
      const size_t off = q_row(a, b, t, hq) * kD + c;
      x = a.q_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(a.q)[off]) : reinterpret_cast<const float*>(a.q)[off];
    }
    reinterpret_cast<float*>(&qt[c][gq >> 2])[gq & 3] = x;
  }
  __syncthreads();
  {
    const int i = i_row;
    float acc[MAXG];
#pragma unroll
    for (int gq = 0; gq < MAXG; ++gq) acc[gq] = 0.f;
#pragma unroll
    for (int j = 0; j < kD / 2; ++j)
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const floatx4 qj = qt[hj * (kD / 2) + j][u];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * u + e] = fmaf(w[j], qj[e], acc[4 * u + e]);
      }
#pragma unroll
    for (int gq = 0; gq < MAXG; ++gq) (hj ? red : qx)[gq][i] = acc[gq];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < MAXG * kD; i += blockDim.x) qx[i / kD][i % kD] += red[i / kD][i % kD];
  __syncthreads();
  // per-head exponent and constants: one wave per head
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int gq = wv; gq < MAXG; gq += 4) {
    // sr: sum of q_rot over the coordinates of the base table; srh over the
    // half-bit coordinates (i mod 32 < 16) of the fractional layout; for the
    // QJL part, sr is sum(q_s)
    float mx = 0.f, sr = 0.f, srh = 0.f;
    for (int c = lane; c < kD; c += 64) {
      const float x = qx[gq][c];
      mx = fmaxf(mx, fabsf(x));
      if (part == 0 && a.key_half && (c & 31) < 16)
        srh += x;
      else
        sr += x;
    }
    mx = wave_max(mx);
    sr = wave_sum(sr);
    srh = wave_sum(srh);
    int ex;
    if (part == 0) {
      float wmax = 0.f;
      for (int p = 0; p < pm; ++p) wmax = fmaxf(wmax, fmaxf(fabsf(a.key_w[p]), fabsf(a.key_w_hi[p])));
      frexpf(mx * wmax, &ex);  // |w_p q_rot| < 2^ex
    } else {
      frexpf(2.f * mx, &ex);
    }
    const int e = 26 - ex;  // scaled values stay below 2^26
    if (lane == 0) {
      e_head[gq] = e;
      if (gq < G) {
        float* cst = a.qconst + ws_row(a, b, h, gq) * 4;
        if (part == 0) {
          cst[0] = a.key_cst * sr + a.key_cst_hi * srh;  // constant part of <q_rot, c[idx]>
          cst[1] = ldexpf(1.f, -e);                      // digit scale of the MSE planes
          if (npl == pm) cst[2] = cst[3] = 0.f;          // no QJL plane
        } else {
          cst[2] = ldexpf(1.f, -e);  // digit scale of the QJL plane
          cst[3] = sr;               // sum(q_s)
        }
      }
    }
  }
  __syncthreads();
  // this part's planes: pl < pm (part 0) or pl == pm (part 1), for every head tile
  const int ppl = part == 0 ? pm : 1;        // planes of this part
  const int ndw = nht * ppl * 2 * 64 * 4;    // their digit dwords
  uint32_t* out = reinterpret_cast<uint32_t*>(a.qdig) + (size_t)(b * a.h_kv + h) * (nht * npl * 2 * 64 * 4);
  for (int i = threadIdx.x; i < ndw; i += blockDim.x) {
    const int d = i & 3;
    const int ln = (i >> 2) & 63;
    const int hf = (i >> 8) & 1;
    const int rest = i >> 9;
    const int pp = rest % ppl, ht = rest / ppl;
    const int pl = part == 0 ? pp : pm;
    const int g = ln >> 4, n = ln & 15;
    const int gq = 4 * ht + (n >> 2), L = n & 3;
    uint32_t word = 0;
    if (gq < G) {
      const int e = e_head[gq];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 32 * g + 8 * j + 4 * hf + d;
        const int s = k & 7;
        // half-bit layout: per-coordinate table; key_w holds zeros past the
        // base table's planes
        const float x = part == 0 ? (a.key_half && (k & 31) < 16 ? a.key_w_hi[pl] : a.key_w[pl]) * qx[gq][k]
                                  : 2.f * qx[gq][k];
        const int q = (int)rintf(ldexpf(x, e - s));
        int dg[4];
        digits128(q, dg);
        const int v = s == 7 ? -dg[L] : dg[L];
        word |= (uint32_t)(v & 0xff) << (8 * j);
      }
    }
    out[((((ht * npl + pl) * 2 + hf) * 64 + ln) << 2) + d] = word;
  }
}

template <int PM, bool QJL, bool VMSE, int PVB, int NHT, bool HALF = false>
__global__ __launch_bounds__(kScanThreads) void scan_mfma_kernel(DecodeArgs a) {
  constexpr int KB = PM == 1 ? 1 : (PM == 2 ? 2 : 3);  // stored key index planes
  constexpr int KP = KB + (QJL ? 1 : 0);               // stored key planes
  // HALF: index plane KB - 1 is the half plane (16-bit chunk per lane group)
  static_assert(!HALF || (QJL && KB >= 2), "the half-bit layout has QJL and a full plane below the half plane");
  constexpr int NPL = PM + (QJL ? 1 : 0);              // score planes
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
  constexpr int kStageTr = VMSE ? 0 : 64 * 16;  // dwords: value-weight digit blocks, exchanged between lanes
  constexpr int kStage = kStageMeta + kStageNg + kStageVw + kStageP + kStageTr;
  constexpr int kMerge = NHEAD * (kD + 2);
  constexpr int kStride = kStage > kMerge ? kStage : kMerge;
  __shared__ __attribute__((aligned(16))) uint32_t smem[4 * kStride];

  // the wave index is uniform: reading it from the first lane keeps the chunk
  // loop, its bounds and the full/partial chunk test in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int sh = blockIdx.y;
  const int b = sh / a.h_kv, h = sh % a.h_kv;
  const int G = a.group;
  const int64_t n_c = a.n_comp.v[b];
  const int64_t t_begin = (int64_t)blockIdx.x * a.split_len;
  const int64_t t_end = t_begin + a.split_len < n_c ? t_begin + a.split_len : n_c;

  uint32_t* s_meta = smem + wave * kStride;
  float* s_ng = reinterpret_cast<float*>(s_meta + kStageMeta);
  uint32_t* s_vw = s_meta + kStageMeta + kStageNg;
  float* s_p = reinterpret_cast<float*>(s_vw + kStageVw);
  uint32_t* s_tr = s_vw + kStageVw + kStageP;

  // query digit operands and per-head constants (score layout: head 4ht + n/4)
  u32x4 qb[NHT][NPL][2];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.qdig) + (size_t)sh * NHT * NPL * 2 * 64;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) qb[ht][pl][hf] = src[((ht * NPL + pl) * 2 + hf) * 64 + lane];
  }
  // score of (head, token) in log2 units: u (K1 Dm + c0) + w (K2 Ds - c3), where
  // u = tau log2(e) n, w = u kappa gamma and Dm, Ds are the digit-combined
  // integer dot products; lane (g, n) scores head 4ht + g
  float k1[NHT], k2[NHT], c0[NHT], c3[NHT], k1h[NHT], k2h[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int hq = 4 * ht + g;
    if (hq < G) {
      const floatx4 cs = *reinterpret_cast<const floatx4*>(a.qconst + ws_row(a, b, h, hq) * 4);
      c0[ht] = cs[0];
      k1[ht] = cs[1];
      k2[ht] = cs[2];
      c3[ht] = cs[3];
    } else {
      c0[ht] = k1[ht] = k2[ht] = c3[ht] = 0.f;
    }
    k1h[ht] = 16384.f * k1[ht];
    k2h[ht] = 16384.f * k2[ht];
  }
  const float u_scale = a.scale * 1.4426950409f;  // exp(x) = exp2(x log2 e)
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

  // key record: full planes of 16 bytes; with HALF the last index plane has 8
  const size_t rec = (size_t)KP * (kD / 8) - (HALF ? kD / 16 : 0);
  const uint8_t* kp = a.k_planes + (size_t)sh * a.capacity * rec;
  const size_t sidx0 = (size_t)sh * a.capacity;
  const uint32_t* vp = a.v_planes + (size_t)sh * (a.capacity >> 5) * VB * kD;

  // running max (log2 units) starts at a finite floor so exp2(-inf - m) is 0, never NaN
  float m_run[NHT], l_part[NHT], acc[NHT][8];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    m_run[ht] = -1e30f;
    l_part[ht] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[ht][nt] = 0.f;
  }

  // Chunk loads are issued one chunk ahead: the registers below hold chunk
  // c0t + 256 of this wave while chunk c0t is being computed.
  uint32_t pX[4][KP];       // key plane words: token 16ct + n, plane word g
  float pNrm = 0.f, pGam = 0.f;
  u32x4 pMeta = u32x4{0u, 0u, 0u, 0u};
  u32x4 pVw[VB];
  const int64_t first = t_begin + 64 * wave;
  const int ssz = a.scalar_f16 ? 2 : 4;
  // Addresses are a wave-uniform chunk base (scalar registers) plus a 32-bit
  // per-lane byte offset, so the loads take the scalar-base form and no
  // 64-bit per-lane pointers stay live across the loop.
  const uint32_t k_lane = n * (uint32_t)rec + 4 * g;  // word g of token n's plane records
  // byte offset of stored plane sp inside a record, for lane group g: full
  // planes at 16 sp + 4g; the half plane's 16-bit chunk g (its coordinates
  // 32g..32g+15) at 16 (KB - 1) + 2g; the QJL plane 8 bytes earlier than a
  // full-plane record would put it
  auto key_off = [&](int sp) -> int {
    if (HALF && sp == KB - 1) return (KB - 1) * (kD / 8) - 2 * g;  // k_lane adds 4g
    if (HALF && sp == KP - 1) return sp * (kD / 8) - kD / 16;
    return sp * (kD / 8);
  };
  auto key_word = [&](const uint8_t* p) -> uint32_t { return *reinterpret_cast<const uint32_t*>(p); };
  auto key_half_word = [&](const uint8_t* p) -> uint32_t { return *reinterpret_cast<const uint16_t*>(p); };
  const uint32_t s_lane = lane * (uint32_t)ssz;       // token `lane`'s scalar
  const uint32_t m_lane = VMSE ? s_lane : lane * (uint32_t)(NG * 4);
  const uint32_t v_lane = lane * 16u;                 // four value words per lane
  auto scalar_at = [&](const void* base, uint32_t off) -> float {
    const char* p = reinterpret_cast<const char*>(base) + off;
    return a.scalar_f16 ? __half2float(*reinterpret_cast<const __half*>(p)) : *reinterpret_cast<const float*>(p);
  };
  auto load_chunk = [&](int it, bool keys, bool rest) {
    const int64_t c = first + (int64_t)it * 256;
    const int rem_c = (int)(t_end - c < 64 ? t_end - c : 64);
    const uint8_t* xk = kp + c * (int64_t)rec;
    const char* xn = reinterpret_cast<const char*>(a.k_norm) + (int64_t)(sidx0 + c) * ssz;
    const char* xg = QJL ? reinterpret_cast<const char*>(a.k_rnorm) + (int64_t)(sidx0 + c) * ssz : nullptr;
    const char* xm = VMSE ? reinterpret_cast<const char*>(a.v_norm) + (int64_t)(sidx0 + c) * ssz
                          : reinterpret_cast<const char*>(a.v_meta) + (int64_t)(sidx0 + c) * (NG * 4);
    const char* xv = reinterpret_cast<const char*>(vp + (c >> 5) * VB * kD);
    if (rem_c == 64 && !rest) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int sp = 0; sp < KP; ++sp)
          pX[ct][sp] = (HALF && sp == KB - 1) ? key_half_word(xk + k_lane + 16 * ct * rec + key_off(sp))
                                               : key_word(xk + k_lane + 16 * ct * rec + key_off(sp));
    } else if (rem_c == 64 && !keys) {
      pNrm = scalar_at(xn, s_lane);
      if (QJL) pGam = scalar_at(xg, s_lane);
      if (VMSE)
        pMeta[0] = __float_as_uint(scalar_at(xm, m_lane));
      else
        pMeta = *reinterpret_cast<const u32x4*>(xm + m_lane);
#pragma unroll
      for (int i = 0; i < VB; ++i) pVw[i] = *reinterpret_cast<const u32x4*>(xv + v_lane + i * 1024);
    } else if (rem_c == 64) {  // full chunk: no per-lane guards
      pNrm = scalar_at(xn, s_lane);
      if (QJL) pGam = scalar_at(xg, s_lane);
      if (VMSE)
        pMeta[0] = __float_as_uint(scalar_at(xm, m_lane));
      else
        pMeta = *reinterpret_cast<const u32x4*>(xm + m_lane);
#pragma unroll
      for (int i = 0; i < VB; ++i) pVw[i] = *reinterpret_cast<const u32x4*>(xv + v_lane + i * 1024);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int sp = 0; sp < KP; ++sp)
          pX[ct][sp] = (HALF && sp == KB - 1) ? key_half_word(xk + k_lane + 16 * ct * rec + key_off(sp))
                                               : key_word(xk + k_lane + 16 * ct * rec + key_off(sp));
    } else {
      const bool valid = lane < rem_c;
      if (rest) {
        pNrm = valid ? scalar_at(xn, s_lane) : 0.f;
        pGam = (QJL && valid) ? scalar_at(xg, s_lane) : 0.f;
        if (VMSE)
          pMeta[0] = valid ? __float_as_uint(scalar_at(xm, m_lane)) : 0u;
        else
          pMeta = valid ? *reinterpret_cast<const u32x4*>(xm + m_lane) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < VB; ++i) {
          const int idx = (i * 64 + lane) * 4;  // dword index inside [2][VB][128]
          pVw[i] = (idx < VB * kD || rem_c > 32) ? *reinterpret_cast<const u32x4*>(xv + v_lane + i * 1024)
                                                 : u32x4{0u, 0u, 0u, 0u};
        }
      }
      if (keys) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const bool v2 = 16 * ct + n < rem_c;
#pragma unroll
          for (int sp = 0; sp < KP; ++sp)
            pX[ct][sp] = !v2 ? 0u
                         : (HALF && sp == KB - 1) ? key_half_word(xk + k_lane + 16 * ct * rec + key_off(sp))
                                                  : key_word(xk + k_lane + 16 * ct * rec + key_off(sp));
        }
      }
    }
  };
  if (first < t_end) load_chunk(0, true, true);

  int it = 0;
  for (int64_t c0t = first; c0t < t_end; c0t += 256, ++it) {
    const int rem = (int)(t_end - c0t < 64 ? t_end - c0t : 64);  // valid tokens of this chunk
    // ---- stage this chunk's per-token data and value words in LDS; the
    // value-weight exponent comes from the largest delta (min/max values) or
    // |v| (MSE values) of the chunk, as bits (non-negative: integer order is
    // float order)
    const uint32_t mb_lane = VMSE ? pMeta[0]
                                  : max(max(pMeta[0] & 0x7fffu, pMeta[1] & 0x7fffu),
                                        max(pMeta[2] & 0x7fffu, pMeta[3] & 0x7fffu));
    // min/max values: the exponent of the value weights is known before the
    // softmax, so p is produced already scaled (see the value section)
    const int ev_mm = VMSE ? 0 : 44 - (int)(wave_max_u32_uniform(mb_lane) >> 10);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    {
      // per token: u, w and an additive mask (-inf past the end of the chunk)
      const float u = u_scale * pNrm;
      *reinterpret_cast<floatx4*>(s_ng + 4 * lane) =
          floatx4{u, QJL ? u * kQjlScale * pGam : 0.f, lane < rem ? 0.f : -INFINITY, 0.f};
      if (VMSE)
        s_meta[lane * NG] = pMeta[0];
      else
        *reinterpret_cast<u32x4*>(s_meta + lane * NG + kMetaPad * (lane >> 4)) = pMeta;
#pragma unroll
      for (int i = 0; i < VB; ++i) {
        const int q = (i * 64 + lane) * 4;  // word index inside the chunk's value words
        *reinterpret_cast<u32x4*>(s_vw + q + kVwPad * (q >> 7)) = pVw[i];
      }
    }
    uint32_t(&X)[4][KP] = pX;  // the key words are reloaded once the scores are done
    if (c0t + 256 < t_end) load_chunk(it + 1, false, true);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    // ---- scores (log2 units).  The query digits are the A operand and the
    // key bits the B operand, so lane (g, n) receives, for token 16ct + n and
    // head 4ht + g, all four digit partial sums (accumulator element r = digit r).
    float sc[NHT][4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      uint32_t P[PM];
      P[0] = X[ct][0];
      if (PM >= 2) P[1 % PM] = X[ct][1 % KP];
      if (PM == 4) {
        P[2 % PM] = X[ct][2 % KP];
        P[3 % PM] = X[ct][0] ^ X[ct][1 % KP] ^ X[ct][2 % KP];
      }
      i32x4 am[NHT], as[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) am[ht] = as[ht] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int pl = 0; pl < PM; ++pl) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x4 Bk = {plane_bytes(P[pl], 4 * hf), plane_bytes(P[pl], 4 * hf + 1),
                            plane_bytes(P[pl], 4 * hf + 2), plane_bytes(P[pl], 4 * hf + 3)};
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) am[ht] = mfma_i8(qb[ht][pl][hf], Bk, am[ht]);
        }
      }
      if (QJL) {
        const uint32_t Ps = X[ct][KP - 1];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x4 Bk = {plane_bytes(Ps, 4 * hf), plane_bytes(Ps, 4 * hf + 1), plane_bytes(Ps, 4 * hf + 2),
                            plane_bytes(Ps, 4 * hf + 3)};
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) as[ht] = mfma_i8(qb[ht][NPL - 1][hf], Bk, as[ht]);
        }
      }
      const int u = 16 * ct + n;  // token inside the chunk
      const floatx4 ng = *reinterpret_cast<const floatx4*>(s_ng + 4 * u);
      const float ut = ng[0], wt = ng[1];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        // digits carry 2^21, 2^14, 2^7, 1: two exact integer halves, each
        // scaled in float (the 2^14 of the upper half is folded into k1h, k2h)
        const float dmh = (float)((am[ht][0] << 7) + am[ht][1]), dml = (float)((am[ht][2] << 7) + am[ht][3]);
        float sv = fmaf(ut, fmaf(dmh, k1h[ht], fmaf(dml, k1[ht], c0[ht])), ng[2]);
        if (QJL) {
          const float dsh = (float)((as[ht][0] << 7) + as[ht][1]), dsl = (float)((as[ht][2] << 7) + as[ht][3]);
          sv = fmaf(wt, fmaf(dsh, k2h[ht], fmaf(dsl, k2[ht], -c3[ht])), sv);
        }
        sc[ht][ct] = sv;
      }
    }
    if (c0t + 64 > lim_min) {  // tail of the compressed part under a causal query
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) sc[ht][ct] = c0t + 16 * ct + n < lim[ht] ? sc[ht][ct] : -INFINITY;
    }

    if (c0t + 256 < t_end) load_chunk(it + 1, true, false);

    // ---- online softmax in log2 units over the 16 lanes of a head (one DPP
    // row); alpha rescales the running sums.  p goes to LDS for the value MFMA,
    // for min/max values as p 2^c with c = ev - 2 min(n/4, 2): token 16ct + n
    // is in slot n/4 of its packed code word, whose bytes carry 4^min(n/4, 2)
    // (4-bit codes: every slot is one whole code per byte, no scale)
    const int c_p = VMSE ? 0 : (VB == 4 ? ev_mm : ev_mm - ((n >> 2) < 2 ? 2 * (n >> 2) : 4));
    float alpha[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const float mloc = row_max16(fmaxf(fmaxf(sc[ht][0], sc[ht][1]), fmaxf(sc[ht][2], sc[ht][3])));
      const float m_new = fmaxf(m_run[ht], mloc);
      alpha[ht] = __builtin_amdgcn_exp2f(m_run[ht] - m_new);
      m_run[ht] = m_new;
      const float m_p = m_new - (float)c_p;
      float lsum = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const float e = __builtin_amdgcn_exp2f(sc[ht][ct] - m_p);  // 0 for tokens past the end
        s_p[(4 * ht + g) * 64 + 16 * ct + n] = e;
        lsum += e;
      }
      l_part[ht] = fmaf(l_part[ht], alpha[ht], VMSE ? lsum : ldexpf(lsum, -c_p));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    float alpha_pv[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) alpha_pv[ht] = alpha[ht];  // accumulator rows: head 4ht + g

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
            V[r] = ((uint32_t)W + 0x00808080u) ^ 0x00808080u;  // bytes = signed base-256 digits
            Mk[k] = fmaf(pe, mn, Mk[k]);
          }
          // 4x4 byte transpose: digit plane d holds byte d of the four tokens
          const uint32_t t01lo = __builtin_amdgcn_perm(V[1], V[0], 0x05010400u);
          const uint32_t t01hi = __builtin_amdgcn_perm(V[1], V[0], 0x07030602u);
          const uint32_t t23lo = __builtin_amdgcn_perm(V[3], V[2], 0x05010400u);
          const uint32_t t23hi = __builtin_amdgcn_perm(V[3], V[2], 0x07030602u);
          A[3][k] = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u);  // least significant digit
          A[2][k] = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u);
          A[1][k] = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u);
          A[0][k] = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);  // most significant digit
        }
        // sum_t p_t min_t per (head, group), the slot scales 2^(ev - 2 min(k, 2))
        // undone: reduce over the four token quarters, then fetch (head g,
        // group gi) for the value layout
        const float x = VB == 4 ? col_sum4(ldexpf((Mk[0] + Mk[1]) + (Mk[2] + Mk[3]), -ev_mm))
                                : col_sum4(ldexpf(fmaf(Mk[0], 1.f, fmaf(Mk[1], 4.f, 16.f * (Mk[2] + Mk[3]))), -ev_mm));
        float Mpv[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) Mpv[gi] = __shfl(x, 4 * g + gi);
        // Exchange the digit blocks inside each quad of lanes: lane (g, 4h + G)
        // holds digit d of row (head h, group G) in A[d]; the value MFMA of
        // group G takes rows (head h, digit d) from lane (g, 4h + d), so one
        // MFMA per channel tile yields all four digits of its own group.  Block
        // d of lane L sits at slot d * 64 + (L ^ d): writes and reads both
        // cover all banks once per 16 lanes.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int d = 0; d < 4; ++d) *reinterpret_cast<u32x4*>(s_tr + 4 * (d * 64 + (lane ^ d))) = A[d];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        u32x4 AG[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          AG[gi] = *reinterpret_cast<const u32x4*>(s_tr + 4 * ((n & 3) * 64 + ((lane & ~3) | (gi ^ (n & 3)))));
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const int gi = nt >> 1;  // group of channels 16nt..16nt+15
          u32x4 B;
          if (VB == 4) {
            // 4-bit codes: tokens 16g..16g+15 are the staged rows 2g and 2g+1
            // (eight tokens each); token i of a word sits in byte i%4, nibble i/4
            const uint32_t w0 = s_vw[(2 * g) * (kD + kVwPad) + 16 * nt + n];
            const uint32_t w1 = s_vw[(2 * g + 1) * (kD + kVwPad) + 16 * nt + n];
            B = u32x4{w0 & 0x0f0f0f0fu, (w0 >> 4) & 0x0f0f0f0fu, w1 & 0x0f0f0f0fu, (w1 >> 4) & 0x0f0f0f0fu};
          } else {
            const uint32_t w = s_vw[g * (kD + kVwPad) + 16 * nt + n];
            B = u32x4{w & 0x03030303u, w & 0x0c0c0c0cu, w & 0x30303030u, (w >> 2) & 0x30303030u};
          }
          // rows (head g, digit r) of group gi: element r is digit r's product
          const i32x4 C = mfma_i8(AG[gi], B, i32x4{0, 0, 0, 0});
          const float v = fmaf((float)((C[0] << 8) + C[1]), 65536.f, (float)((C[2] << 8) + C[3]));
          acc[ht][nt] = fmaf(acc[ht][nt], alpha_pv[ht], fmaf(v, inv_sv, Mpv[gi]));
        }
      }
    } else {
      // this lane's 16 tokens in the bit-plane order: 16ct + 4g + r
      floatx4 pv[NHT][4];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          pv[ht][ct] = *reinterpret_cast<const floatx4*>(s_p + (4 * ht + (n >> 2)) * 64 + 16 * ct + 4 * g);
      // MSE values: weights p_t |v_t| (same for every value plane), rows (head,
      // digit); accumulated in rotated space
      const int mydig_shift = 7 * (3 - (n & 3));
      const uint32_t mb = wave_max_u32_uniform(mb_lane);
      int ex;
      frexpf(__uint_as_float(mb), &ex);
      const int ev = 26 - ex;
      const float inv_sv = ldexpf(1.f, -ev);
      u32x4 A[NHT];
      float PN[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        A[ht] = u32x4{0u, 0u, 0u, 0u};
        PN[ht] = 0.f;
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int s_tok = 4 * (ct & 1) + g;
        const float sc = ldexpf(1.f, ev - s_tok);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int u = 16 * ct + 4 * g + r;
          const float nv = __uint_as_float(s_meta[u * NG]);
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) {
            const uint32_t W = (uint32_t)fmaf(pv[ht][ct][r], nv * sc, 0.5f);
            int dg = (int)((W >> mydig_shift) & 127u);
            if (s_tok == 7) dg = -dg;
            A[ht][ct] |= (uint32_t)(dg & 0xff) << (8 * r);
            PN[ht] = fmaf(pv[ht][ct][r], nv, PN[ht]);
          }
        }
      }
      float PNpv[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const float x = col_sum4(PN[ht]);
        PNpv[ht] = __shfl(x, 4 * g);
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
#pragma unroll
        for (int pl = 0; pl < PVB; ++pl) {
          u32x4 B;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t w = pl < VB ? Wd[d][pl % VB] : (Wd[d][0] ^ Wd[d][1 % VB] ^ Wd[d][2 % VB]);
            B[d] = plane_bytes(w, 4 * (d & 1) + g);
          }
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) {
            const i32x4 C = mfma_i8(A[ht], B, i32x4{0, 0, 0, 0});
            const int hi = (C[0] << 7) + C[1], lo = (C[2] << 7) + C[3];
            const float v = fmaf((float)hi, 16384.f, (float)lo);
            vs[ht] = fmaf(v, a.val_w[pl], vs[ht]);
          }
        }
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          acc[ht][nt] = fmaf(acc[ht][nt], alpha_pv[ht], fmaf(vs[ht], inv_sv, a.val_cst * PNpv[ht]));
      }
    }
  }

  // ---- merge the four waves: one (m, l, acc[128]) partial per query head,
  // with m converted back to natural-log units
  float lsum[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) lsum[ht] = row_sum16(l_part[ht]);  // the 16 lanes of head 4ht + g
  __syncthreads();
  float* mrg = reinterpret_cast<float*>(smem) + wave * kStride;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    if (n == 0) {
      const int hh = 4 * ht + g;
      mrg[hh * (kD + 2)] = lsum[ht] > 0.f ? m_run[ht] * 0.6931471806f : -INFINITY;
      mrg[hh * (kD + 2) + 1] = lsum[ht];
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) mrg[(4 * ht + g) * (kD + 2) + 2 + 16 * nt + n] = acc[ht][nt];
  }
  __syncthreads();
  const float* base = reinterpret_cast<const float*>(smem);
  for (int i = threadIdx.x; i < G * kD; i += blockDim.x) {
    const int hh = i / kD, c = i % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, base[w * kStride + hh * (kD + 2)]);
    float L = 0.f, Acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = base[w * kStride + hh * (kD + 2)];
        const float f = mw == -INFINITY ? 0.f : __expf(mw - M);
        L += f * base[w * kStride + hh * (kD + 2) + 1];
        Acc += f * base[w * kStride + hh * (kD + 2) + 2 + c];
      }
    }
    float* part = a.partial + ((size_t)blockIdx.x * a.batch * a.h_kv * G + ws_row(a, b, h, hh)) * (kD + 2);
    if (c == 0) {
      part[0] = M;
      part[1] = L;
    }
    part[2 + c] = Acc;
  }
}

template <int PM, bool QJL, bool VMSE, int PVB, int NHT, bool HALF = false>
hipError_t launch_scan_mfma(const DecodeArgs& a, hipStream_t st, TimedLaunch tl) {
  if (tl.begin) (void)hipEventRecord(tl.begin, st);
  hipLaunchKernelGGL((scan_mfma_kernel<PM, QJL, VMSE, PVB, NHT, HALF>), dim3(a.splits, a.batch * a.h_kv),
                     dim3(kScanThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (tl.end) (void)hipEventRecord(tl.end, st);
  return e;
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

size_t mfma_workspace_bytes(int batch, int h_q, int group) {
  const int nht = (group + 3) / 4;
  const int h_kv = h_q / group;
  const size_t dig = (size_t)batch * h_kv * nht * 5 * 2 * 64 * 16;  // up to 5 score planes
  const size_t cst = (size_t)batch * h_q * 4 * 4;
  return dig + cst + 256;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int key_mse_bits, int key_qjl, int value_mse,
                              int value_bits, int key_planes, int value_planes, hipStream_t stream,
                              TimedLaunch tl) {
  // covered: keys with 1-, 2- or 3-bit indices (or 1.5 / 2.5 with QJL), with
  // or without the QJL bit, 2- or 4-bit min/max values in groups of 32 or
  // 3-bit MSE values (2-bit MSE values with 2+1- and 3+1-bit keys),
  // antisymmetric codebooks, up to 8 query heads per KV head
  if (key_mse_bits < 1 || key_mse_bits > 3) return hipErrorNotSupported;
  if (!key_qjl && a.key_half) return hipErrorNotSupported;
  if (key_planes != (1 << (key_mse_bits - 1))) return hipErrorNotSupported;
  if (value_mse) {
    if ((value_bits != 2 && value_bits != 3) || value_planes != (1 << (value_bits - 1))) return hipErrorNotSupported;
    if (value_bits == 2 && (!key_qjl || a.key_half || key_mse_bits < 2)) return hipErrorNotSupported;
  } else if ((value_bits != 2 && value_bits != 4) || a.value_group != 32) {
    return hipErrorNotSupported;
  }
  if (a.group > 8) return hipErrorNotSupported;
  const int nht = a.group > 4 ? 2 : 1;
  const int pm = 1 << (key_mse_bits - 1);
  const int npl = pm + (key_qjl ? 1 : 0);
  const dim3 qgrid(a.batch * a.h_kv, key_qjl ? 2 : 1);
  if (nht == 1)
    hipLaunchKernelGGL(qprep_mfma_kernel<4>, qgrid, dim3(256), 0, stream, a, pm, npl, nht);
  else
    hipLaunchKernelGGL(qprep_mfma_kernel<8>, qgrid, dim3(256), 0, stream, a, pm, npl, nht);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = nht == 1 ? dispatch_mfma<1>(a, key_mse_bits, key_qjl, value_mse, value_bits, stream, tl)
               : dispatch_mfma<2>(a, key_mse_bits, key_qjl, value_mse, value_bits, stream, tl);
  if (e != hipSuccess) return e;
  return launch_combine(a, value_mse, stream);
}

}  // namespace tq
