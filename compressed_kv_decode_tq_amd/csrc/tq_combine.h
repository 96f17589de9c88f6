// Split combine and ring merge of one (sequence, KV head, virtual head): the
// last step of a decode (page "03. Results & Benchmarks", "Latency
// Benchmarks": the online softmax over all tokens; page "turboquant/
// audit_claims.py", AUDIT 1: the recent tokens kept uncompressed in a bf16
// ring, attended exactly).
//
// A combine unit is 128 threads, thread c owning output channel c.  Every
// barrier below is a whole-work-group barrier executed unconditionally (a unit
// with no head to combine still takes part in the barriers).
#pragma once

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {


// LDS of one combine unit for at most MAXS splits.
template <int MAXS>
struct CombineLds {
  float qv[kD];
  float s_f[MAXS];  // per split: m, then its merge factor
  float s_l[MAXS];
  float pr[kD];     // ring probabilities (ring_cap <= 128 per pass)
  float arot[kD];
  float red[2];
};

// Max / sum over the two waves of a unit, result in every thread of the unit.
__device__ __forceinline__ float unit_max(float x, float* red) {
  x = wave_max(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[(threadIdx.x >> 6) & 1] = x;
  __syncthreads();
  return fmaxf(red[0], red[1]);
}
__device__ __forceinline__ float unit_sum(float x, float* red) {
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[(threadIdx.x >> 6) & 1] = x;
  __syncthreads();
  return red[0] + red[1];
}

// Merge of the split partials (m, l, acc) of virtual head gq of slot (b, h),
// split s at part0 + s * sstride (global memory, or LDS for one split), with
// the exact ring tokens; MSE values (VMSE) are rotated back with Pi^T
// once.  Writes out[.][c].  Every load that needs no earlier result (split
// headers, the first kCombinePre splits' acc words, the ring key row, the
// first kRingPre ring values) is issued before its first use, so the merge
// costs about one memory round trip.  `active` false: no head for this unit,
// barriers only.  a.splits <= MAXS.
template <bool VMSE, int MAXS>
__device__ __forceinline__ void combine_unit(const DecodeArgs& a, int b, int h, int gq, bool active,
                                             CombineLds<MAXS>& L, const float* part0, size_t sstride) {
  constexpr int kCombinePre = 16;  // splits whose accumulator word is loaded up front
  constexpr int kRingPre = 32;     // ring values loaded up front
  const int c = threadIdx.x & (kD - 1);
  int t = 0, hq = 0, nr = 0, S = 0;
  if (active) {
    int hide_c, hide_r;
    virtual_head(a, h, gq, t, hq);
    hidden_keys(a, t, (int)a.n_ring.v[b], hide_c, hide_r);
    nr = (int)a.n_ring.v[b] - hide_r;  // ring tokens this query sees
    S = a.splits;
  }
  const size_t ring_row = (size_t)b * a.ring_cap * a.h_kv + h;  // ring token j: (ring_row + j h_kv) kD

  // ---- loads
  float qc = 0.f;
  if (active) {
    const size_t qoff = q_row(a, b, t, hq) * kD + c;
    qc = a.q_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(a.q)[qoff]) : reinterpret_cast<const float*>(a.q)[qoff];
  }
  float hm = -INFINITY, hl = 0.f;  // header of split c (thread c < S)
  if (c < S) {
    hm = part0[(size_t)c * sstride];
    hl = part0[(size_t)c * sstride + 1];
  }
  float pa[kCombinePre];
#pragma unroll
  for (int u = 0; u < kCombinePre; ++u) pa[u] = u < S ? part0[(size_t)u * sstride + 2 + c] : 0.f;
  u32x4 kw[kD / 8];  // thread j's ring token key row (256 bytes)
  if (c < nr) {
    const u32x4* kr = reinterpret_cast<const u32x4*>(a.ring_k + (ring_row + (size_t)c * a.h_kv) * kD);
#pragma unroll
    for (int i = 0; i < kD / 8; ++i) kw[i] = kr[i];
  }
  float rv[kRingPre];
#pragma unroll
  for (int u = 0; u < kRingPre; ++u)
    rv[u] = u < nr ? bf2f(a.ring_v[(ring_row + (size_t)u * a.h_kv) * kD + c]) : 0.f;

  // ---- split headers (m, l): thread c takes splits c, c + 128, ...
  L.qv[c] = qc;
  float M = hm;
  if (c < S) {
    L.s_f[c] = hm;
    L.s_l[c] = hl;
  }
  for (int sp = c + kD; sp < S; sp += kD) {
    const float* ph = part0 + (size_t)sp * sstride;
    const float m = ph[0], l = ph[1];
    L.s_f[sp] = m;
    L.s_l[sp] = l;
    M = fmaxf(M, m);
  }
  __syncthreads();  // qv

  // ring scores: thread j scores ring token j
  float sj = -INFINITY;
  if (c < nr) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kD / 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(L.qv[8 * i + 2 * e], bf2f(kw[i][e] & 0xffffu), acc);
        acc = fmaf(L.qv[8 * i + 2 * e + 1], bf2f(kw[i][e] >> 16), acc);
      }
    sj = a.scale * acc;
  }
  M = unit_max(fmaxf(M, sj), L.red);
  const bool any = M != -INFINITY;  // uniform over the unit; false: no token at all

  // merge factors of the splits and of the ring tokens; L in one unit sum
  float Lp = 0.f;
  if (any) {
    for (int sp = c; sp < S; sp += kD) {
      const float m = L.s_f[sp];
      const float f = m == -INFINITY ? 0.f : __expf(m - M);
      L.s_f[sp] = f;
      Lp = fmaf(f, L.s_l[sp], Lp);
    }
  }
  const float pj = (any && c < nr) ? __expf(sj - M) : 0.f;
  L.pr[c] = pj;
  const float Lsum = unit_sum(Lp + pj, L.red);  // its barriers also publish s_f and pr

  // channel c: sum over splits of f_s acc_s[c]; splits past the first
  // kCombinePre are loaded sixteen at a time
  float A = 0.f;
  if (any) {
#pragma unroll
    for (int u = 0; u < kCombinePre; ++u)
      if (u < S) A = fmaf(L.s_f[u], pa[u], A);
    constexpr int kBatch = 16;  // split accumulator words per round of loads
    int sp = kCombinePre;
#pragma unroll 1
    for (; sp + kBatch <= S; sp += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = part0[(size_t)(sp + u) * sstride + 2 + c];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) A = fmaf(L.s_f[sp + u], v[u], A);
    }
    for (; sp < S; ++sp) A = fmaf(L.s_f[sp], part0[(size_t)sp * sstride + 2 + c], A);
  }
  if (VMSE) {  // accumulated in rotated space: apply Pi^T once (column c of Pi)
    L.arot[c] = A;
    __syncthreads();
    if (any) {
      float o = 0.f;
#pragma unroll 1
      for (int i0 = 0; i0 < kD; i0 += 16) {
        float w[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) w[u] = a.pi[(size_t)(i0 + u) * kD + c];
#pragma unroll
        for (int u = 0; u < 16; ++u) o = fmaf(w[u], L.arot[i0 + u], o);
      }
      A = o;
    }
  }
  if (any) {
    // ring values (original space): the first kRingPre are in registers, the
    // rest come 32 loads at a time
#pragma unroll
    for (int u = 0; u < kRingPre; ++u) A = fmaf(u < nr ? L.pr[u] : 0.f, rv[u], A);
    constexpr int kRingBatch = 32;  // ring values per round of loads
#pragma unroll 1
    for (int j0 = kRingPre; j0 < nr; j0 += kRingBatch) {
      float v[kRingBatch];
#pragma unroll
      for (int u = 0; u < kRingBatch; ++u)
        v[u] = j0 + u < nr ? bf2f(a.ring_v[(ring_row + (size_t)(j0 + u) * a.h_kv) * kD + c]) : 0.f;
#pragma unroll
      for (int u = 0; u < kRingBatch; ++u) A = fmaf(j0 + u < nr ? L.pr[j0 + u] : 0.f, v[u], A);
    }
  }
  if (active) a.out[q_row(a, b, t, hq) * kD + c] = (any && Lsum > 0.f) ? A / Lsum : 0.f;
}

}  // namespace tq
