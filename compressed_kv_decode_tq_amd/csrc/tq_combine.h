// Split combine and ring merge of one (sequence, KV head, virtual head): the
// last step of a decode (page "03. Results & Benchmarks", "Latency
// Benchmarks": the online softmax over all tokens; page "turboquant/
// audit_claims.py", AUDIT 1: the recent tokens kept uncompressed in a bf16
// ring, attended exactly).
//
// A combine unit is one work-group of 512 threads.  Thread (qq, c) = (tid / 128,
// tid % 128) owns output channel c for quarter qq of the splits, of the ring
// tokens and (MSE values) of the rows of Pi; the four quarters meet in LDS.
// Ring token j is scored by the four threads 4j .. 4j + 3 (32 channels each,
// one DPP quad sum), so its key row is read as one contiguous 256-byte block.
// Every barrier below is a whole-work-group barrier executed unconditionally.
#pragma once

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {

constexpr int kCombineThreads = 512;
constexpr int kCombineQuarters = kCombineThreads / kD;

// LDS of one combine unit for at most MAXS splits.
template <int MAXS>
struct CombineLds {
  float qv[kD];
  float s_f[MAXS];  // per split: m, then its merge factor
  float s_l[MAXS];
  float pr[kMaxRing];                // ring probabilities
  float part[kCombineQuarters][kD];  // per-quarter channel sums
  float arot[kD];
  float red[kCombineThreads / 64];
};

// Sum over the 4 lanes of a quad (xor 1, then xor 2) with DPP.
__device__ __forceinline__ float combine_quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
  return x;
}

// Max / sum over the work-group's waves, result in every thread.
__device__ __forceinline__ float unit_max(float x, float* red) {
  x = wave_max(x);
  __syncthreads();  // red is free again
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}
__device__ __forceinline__ float unit_sum(float x, float* red) {
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) r += red[w];
  return r;
}

// Merge of the split partials (m, l, acc) of virtual head gq of slot (b, h),
// split s at part0 + s * sstride, with the exact ring tokens; MSE values (VMSE)
// are rotated back with Pi^T once.  Writes out[.][c].  The loads that need no
// earlier result (split headers, each quarter's first kPre split words, the
// ring key rows, each quarter's first kRingPre ring values and, for MSE
// values, each quarter's rows of Pi) are issued before their first use.
// a.splits <= MAXS; at most kMaxRing ring tokens.  PRE: split accumulator
// words per thread loaded up front (each quarter's first PRE splits; the rest
// come kBatch at a time).
template <bool VMSE, int MAXS, int PRE>
__device__ __forceinline__ void combine_unit(const DecodeArgs& a, int b, int h, int gq, CombineLds<MAXS>& L,
                                             const float* part0, size_t sstride) {
  constexpr int Q = kCombineQuarters;
  constexpr int kPre = PRE;
  constexpr int kRingPre = 8;  // ring values per thread loaded up front
  constexpr int kBatch = 8;    // loads per later round
  const int tid = threadIdx.x, c = tid & (kD - 1), qq = tid / kD;
  int t, hq, hide_c, hide_r;
  virtual_head(a, h, gq, t, hq);
  hidden_keys(a, t, (int)a.n_ring.v[b], hide_c, hide_r);
  const int nr = (int)a.n_ring.v[b] - hide_r;  // ring tokens this query sees
  const int S = a.splits;
  const size_t ring_row = (size_t)b * a.ring_cap * a.h_kv + h;  // ring token j: (ring_row + j h_kv) kD

  // ---- loads, all issued before the first is used: raw bits, converted where
  // they are used, so no conversion waits on a load while later loads are
  // still to be issued
  const size_t qoff = q_row(a, b, t, hq) * kD + c;
  uint32_t qraw = 0u;
  if (tid < kD)
    qraw = a.q_bf16 ? (uint32_t)reinterpret_cast<const uint16_t*>(a.q)[qoff]
                    : reinterpret_cast<const uint32_t*>(a.q)[qoff];
  constexpr int kHdr = (MAXS + kCombineThreads - 1) / kCombineThreads;  // split headers per thread
  float hm[kHdr], hl[kHdr];  // thread tid takes splits tid, tid + 512, ...
#pragma unroll
  for (int u = 0; u < kHdr; ++u) {
    const int sp = tid + kCombineThreads * u;
    hm[u] = sp < S ? part0[(size_t)sp * sstride] : -INFINITY;
    hl[u] = sp < S ? part0[(size_t)sp * sstride + 1] : 0.f;
  }
  float pa[kPre];  // quarter qq: splits qq, qq + 4, ...
#pragma unroll
  for (int u = 0; u < kPre; ++u) pa[u] = qq + Q * u < S ? part0[(size_t)(qq + Q * u) * sstride + 2 + c] : 0.f;
  const int rj = tid >> 2, rq = tid & 3;  // ring token scored, and its channel quarter
  u32x4 kw[4];
  if (rj < nr) {
    const u32x4* kr = reinterpret_cast<const u32x4*>(a.ring_k + (ring_row + (size_t)rj * a.h_kv) * kD + 32 * rq);
#pragma unroll
    for (int i = 0; i < 4; ++i) kw[i] = kr[i];
  }
  // quarter qq: ring tokens qq, qq + 4, ... (bf16 bits), read from tokens
  // clamped to the last one seen (the extra values are never used) by the
  // waves whose quarter has a token at all (the quarter is uniform over a wave)
  uint32_t rv[kRingPre] = {};
  if (__builtin_amdgcn_readfirstlane(qq) < nr) {
#pragma unroll
    for (int u = 0; u < kRingPre; ++u)
      rv[u] = a.ring_v[(ring_row + (size_t)min(qq + Q * u, nr - 1) * a.h_kv) * kD + c];
  }
  // MSE values: column c of Pi, rows (kD / Q) qq .. + kD / Q - 1 (the
  // rotation back of this quarter's part of the merged accumulator)
  float wpi[VMSE ? kD / Q : 1];
  if (VMSE) {
#pragma unroll
    for (int u = 0; u < kD / Q; ++u) wpi[u] = a.pi[(size_t)((kD / Q) * qq + u) * kD + c];
  }
  if (tid < kD) L.qv[c] = a.q_bf16 ? bf2f(qraw) : __uint_as_float(qraw);
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kHdr; ++u) {
    const int sp = tid + kCombineThreads * u;
    if (sp < S) {
      L.s_f[sp] = hm[u];
      L.s_l[sp] = hl[u];
    }
    M = fmaxf(M, hm[u]);
  }
  __syncthreads();  // qv, split headers

  // ---- ring scores
  float sj = -INFINITY;
  {
    float acc = 0.f;
    if (rj < nr) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = fmaf(L.qv[32 * rq + 8 * i + 2 * e], bf2f(kw[i][e] & 0xffffu), acc);
          acc = fmaf(L.qv[32 * rq + 8 * i + 2 * e + 1], bf2f(kw[i][e] >> 16), acc);
        }
    }
    acc = combine_quad_sum(acc);  // the token's four threads are one quad of a wave
    if (rj < nr) sj = a.scale * acc;
  }
  M = unit_max(fmaxf(M, sj), L.red);
  const bool any = M != -INFINITY;  // uniform over the unit; false: no token at all

  // merge factors of the splits and of the ring tokens; L in one unit sum
  float Lp = 0.f;
  if (any) {
    for (int sp = tid; sp < S; sp += kCombineThreads) {
      const float m = L.s_f[sp];
      const float f = m == -INFINITY ? 0.f : __expf(m - M);
      L.s_f[sp] = f;
      Lp = fmaf(f, L.s_l[sp], Lp);
    }
  }
  const float pj = (any && rj < nr) ? __expf(sj - M) : 0.f;
  if (rq == 0) L.pr[rj] = pj;  // rj < 128 = kMaxRing
  const float Lsum = unit_sum(Lp + (rq == 0 ? pj : 0.f), L.red);  // its barriers also publish s_f and pr

  // ---- channel c, quarter qq of the splits
  float A = 0.f;
  if (any) {
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      if (qq + Q * u < S) A = fmaf(L.s_f[qq + Q * u], pa[u], A);
    int u0 = kPre;
#pragma unroll 1
    for (; qq + Q * (u0 + kBatch - 1) < S; u0 += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = part0[(size_t)(qq + Q * (u0 + u)) * sstride + 2 + c];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) A = fmaf(L.s_f[qq + Q * (u0 + u)], v[u], A);
    }
    for (int sp = qq + Q * u0; sp < S; sp += Q) A = fmaf(L.s_f[sp], part0[(size_t)sp * sstride + 2 + c], A);
  }
  if (VMSE) {  // accumulated in rotated space: apply Pi^T once (column c of Pi, rows of quarter qq)
    L.part[qq][c] = A;
    __syncthreads();
    if (tid < kD) L.arot[c] = (L.part[0][c] + L.part[1][c]) + (L.part[2][c] + L.part[3][c]);
    __syncthreads();  // arot written, part read: part is free again
    float o = 0.f;
    if (any) {
#pragma unroll
      for (int u = 0; u < kD / Q; ++u) o = fmaf(wpi[u], L.arot[(kD / Q) * qq + u], o);
    }
    A = o;
  }
  if (any) {
    // ring values (original space), quarter qq of the ring tokens: the first
    // kRingPre are in registers, the rest come kBatch loads at a time
#pragma unroll
    for (int u = 0; u < kRingPre; ++u)
      if (qq + Q * u < nr) A = fmaf(L.pr[qq + Q * u], bf2f(rv[u]), A);
#pragma unroll 1
    for (int u0 = kRingPre; qq + Q * u0 < nr; u0 += kBatch) {
      uint32_t v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = min(qq + Q * (u0 + u), nr - 1);
        v[u] = a.ring_v[(ring_row + (size_t)j * a.h_kv) * kD + c];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = qq + Q * (u0 + u);
        if (j < nr) A = fmaf(L.pr[j], bf2f(v[u]), A);
      }
    }
  }
  L.part[qq][c] = A;
  __syncthreads();
  if (tid < kD) {
    const float tot = (L.part[0][c] + L.part[1][c]) + (L.part[2][c] + L.part[3][c]);
    a.out[q_row(a, b, t, hq) * kD + c] = (any && Lsum > 0.f) ? tot / Lsum : 0.f;
  }
}

}  // namespace tq
