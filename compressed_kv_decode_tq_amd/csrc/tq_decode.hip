// Decode kernels for gfx950: query preparation, the split scan over the
// compressed cache, and the split combine with the ring merge.
//
// Method (page "03. Results & Benchmarks", section "Latency Benchmarks": scores,
// QJL correction, online softmax and value accumulation in one pass; page
// "TurboQuant — Random rotation trước khi quantize, 3-bit KV cache không mất
// accuracy", section "Tại sao nó hoạt động": the query is rotated once per step
// and keys are never reconstructed).  For query head hq of KV head h:
//   q_rot = Pi q, q_s = S q
//   s_j   = tau n_j ( <q_rot, c[idx_j]> + sqrt(pi/2)/d gamma_j <q_s, sigma_j> )
//   o     = sum_j p_j v~_j / sum_j p_j over compressed and ring tokens, where
//           v~_j = min_j + delta_j code_j (min/max values) or, for MSE values,
//           the accumulation runs in rotated space and Pi^T is applied once.
#include "tq_combine.h"
#include "tq_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kScanThreads = 256;  // 4 waves, each taking 64-token chunks of the split
constexpr int kChunk = 64;
constexpr float kQjlScale = 0.0097916519f;  // sqrt(pi/2) / 128

// q_rot = Pi q and q_s = S q for the G (virtual) heads of one (sequence, KV head).
__global__ __launch_bounds__(256) void qprep_kernel(DecodeArgs a) {
  __shared__ float qv[kMaxGroup][kD];
  const int b = blockIdx.x / a.h_kv, h = blockIdx.x % a.h_kv;
  const int G = a.group;
  for (int i = threadIdx.x; i < G * kD; i += blockDim.x) {
    const int c = i % kD;
    int t, hq;
    virtual_head(a, h, i / kD, t, hq);
    const size_t off = q_row(a, b, t, hq) * kD + c;
    qv[i / kD][c] = a.q_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(a.q)[off])
                             : reinterpret_cast<const float*>(a.q)[off];
  }
  __syncthreads();
  const int i = threadIdx.x & (kD - 1);
  const int which = threadIdx.x >> 7;  // 0: Pi, 1: S
  const float* m = which == 0 ? a.pi : a.s;
  float acc[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) acc[g] = 0.f;
  const floatx4* row = reinterpret_cast<const floatx4*>(m + (size_t)i * kD);
  for (int j4 = 0; j4 < kD / 4; ++j4) {
    const floatx4 w = row[j4];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
      if (g < G) {
        acc[g] = fmaf(w[0], qv[g][4 * j4 + 0], acc[g]);
        acc[g] = fmaf(w[1], qv[g][4 * j4 + 1], acc[g]);
        acc[g] = fmaf(w[2], qv[g][4 * j4 + 2], acc[g]);
        acc[g] = fmaf(w[3], qv[g][4 * j4 + 3], acc[g]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g)
    if (g < G) a.qprep[(ws_row(a, b, h, g) * 2 + which) * kD + i] = acc[g];
}

// Split scan: work-group (split, sequence*KV head).  Lane = token for the
// scores, lane = two channels for the value accumulation.
template <int KB, bool QJL, bool VMSE, int VB>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(DecodeArgs a) {
  constexpr int KP = KB + (QJL ? 1 : 0);
  __shared__ __attribute__((aligned(16))) float qr[kD][kMaxGroup];  // [coordinate][head]
  __shared__ __attribute__((aligned(16))) float qs[kD][kMaxGroup];
  __shared__ __attribute__((aligned(16))) float pb[4][kChunk][kMaxGroup];  // p per wave, token, head
  __shared__ __attribute__((aligned(16))) uint32_t mb[4][kChunk][8];     // value meta per token
  __shared__ float kc[16], vc[16];
  __shared__ float mrg[4][kMaxGroup][2];

  const int split = blockIdx.x;
  const int sh = blockIdx.y;  // b * h_kv + h
  const int b = sh / a.h_kv, h = sh % a.h_kv;
  const int G = a.group;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n_c = a.n_comp.v[b];
  const int64_t t_begin = (int64_t)split * a.split_len;
  const int64_t t_end = t_begin + a.split_len < n_c ? t_begin + a.split_len : n_c;

  for (int i = threadIdx.x; i < kD * kMaxGroup; i += blockDim.x) {
    const int c = i / kMaxGroup, g = i % kMaxGroup;
    const size_t base = ws_row(a, b, h, g < G ? g : 0) * 2 * kD;
    qr[c][g] = g < G ? a.qprep[base + c] : 0.f;
    qs[c][g] = g < G ? a.qprep[base + kD + c] : 0.f;
  }
  if (threadIdx.x < 16) {
    kc[threadIdx.x] = a.k_cent[threadIdx.x];
    vc[threadIdx.x] = a.v_cent[threadIdx.x];
  }
  __syncthreads();

  const size_t rec = (size_t)KP * (kD / 8);
  const uint8_t* kp = a.k_planes + (size_t)sh * key_slot_tokens(a.capacity) * rec;
  const size_t sidx0 = (size_t)sh * a.capacity;
  const int ngrp = kD / a.value_group;
  const uint32_t* vp = a.v_planes + (size_t)sh * (a.capacity >> 5) * VB * kD;

  // compressed tokens each (virtual) head sees: all of them for one query per
  // sequence, fewer for the earlier of several causal queries
  int64_t lim[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    int t, hq, hide_c, hide_r;
    virtual_head(a, h, g, t, hq);
    hidden_keys(a, t, (int)a.n_ring.v[b], hide_c, hide_r);
    lim[g] = n_c - hide_c;
  }
  float m_run[kMaxGroup], l_part[kMaxGroup], acc0[kMaxGroup], acc1[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    m_run[g] = -INFINITY;
    l_part[g] = 0.f;
    acc0[g] = 0.f;
    acc1[g] = 0.f;
  }

  const int64_t span = t_end > t_begin ? t_end - t_begin : 0;
  const int iters = (int)((span + 4 * kChunk - 1) / (4 * kChunk));
  for (int it = 0; it < iters; ++it) {
    const int64_t c0 = t_begin + ((int64_t)it * 4 + wave) * kChunk;  // chunk start (multiple of 64)
    // ---- scores: lane = token
    const int64_t tok = c0 + lane;
    const bool valid = tok < t_end;
    float s[kMaxGroup];
    {
      uint32_t w[KP][4];
      float n = 0.f, gam = 0.f;
      if (valid) {
#pragma unroll
        for (int p = 0; p < KP; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) w[p][e] = *reinterpret_cast<const uint32_t*>(kp + key_word_offset(tok, rec, p * 16, e, 4));
        n = load_scalar(a.k_norm, sidx0 + tok, a.scalar_f16);
        if (QJL) gam = load_scalar(a.k_rnorm, sidx0 + tok, a.scalar_f16);
      } else {
#pragma unroll
        for (int p = 0; p < KP; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) w[p][e] = 0u;
      }
      float dm[kMaxGroup], dq[kMaxGroup];
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g) dm[g] = dq[g] = 0.f;
#pragma unroll 4
      for (int i = 0; i < kD; ++i) {
        int idx = 0;
#pragma unroll
        for (int p = 0; p < KB; ++p) idx |= (int)((w[p][i >> 5] >> (i & 31)) & 1u) << p;
        const float c = kc[idx];
        const floatx4 q0 = *reinterpret_cast<const floatx4*>(&qr[i][0]);
        const floatx4 q1 = *reinterpret_cast<const floatx4*>(&qr[i][4]);
        dm[0] = fmaf(q0[0], c, dm[0]);
        dm[1] = fmaf(q0[1], c, dm[1]);
        dm[2] = fmaf(q0[2], c, dm[2]);
        dm[3] = fmaf(q0[3], c, dm[3]);
        if (G > 4) {
          dm[4] = fmaf(q1[0], c, dm[4]);
          dm[5] = fmaf(q1[1], c, dm[5]);
          dm[6] = fmaf(q1[2], c, dm[6]);
          dm[7] = fmaf(q1[3], c, dm[7]);
        }
        if (QJL) {
          const float sg = ((w[KB][i >> 5] >> (i & 31)) & 1u) ? 1.f : -1.f;
          const floatx4 r0 = *reinterpret_cast<const floatx4*>(&qs[i][0]);
          const floatx4 r1 = *reinterpret_cast<const floatx4*>(&qs[i][4]);
          dq[0] = fmaf(r0[0], sg, dq[0]);
          dq[1] = fmaf(r0[1], sg, dq[1]);
          dq[2] = fmaf(r0[2], sg, dq[2]);
          dq[3] = fmaf(r0[3], sg, dq[3]);
          if (G > 4) {
            dq[4] = fmaf(r1[0], sg, dq[4]);
            dq[5] = fmaf(r1[1], sg, dq[5]);
            dq[6] = fmaf(r1[2], sg, dq[6]);
            dq[7] = fmaf(r1[3], sg, dq[7]);
          }
        }
      }
      const float kg = kQjlScale * gam;
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g) s[g] = valid && tok < lim[g] ? a.scale * n * (dm[g] + kg * dq[g]) : -INFINITY;
    }
    // ---- online softmax update (every lane of the wave holds the same m_run)
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
      if (g >= G) break;
      const float cmax = wave_max(s[g]);
      const float m_new = fmaxf(m_run[g], cmax);
      const float alpha = m_run[g] == -INFINITY ? 0.f : __expf(m_run[g] - m_new);
      const float p = s[g] != -INFINITY ? __expf(s[g] - m_new) : 0.f;  // masked: 0
      m_run[g] = m_new;
      l_part[g] = l_part[g] * alpha + p;
      acc0[g] *= alpha;
      acc1[g] *= alpha;
      pb[wave][lane][g] = p;
    }
    // stage value metadata of the chunk's tokens (zeros for tokens past the end)
    if (VMSE) {
      mb[wave][lane][0] = valid ? __float_as_uint(load_scalar(a.v_norm, sidx0 + tok, a.scalar_f16)) : 0u;
    } else {
      const uint32_t* mp = reinterpret_cast<const uint32_t*>(a.v_meta) + (sidx0 + tok) * ngrp;
      for (int gi = 0; gi < ngrp; ++gi) mb[wave][lane][gi] = valid ? mp[gi] : 0u;
    }
    __syncthreads();  // every wave runs the same number of iterations
    // ---- values: lane = channels 2*lane, 2*lane+1
    {
      const int ch = 2 * lane;
      uint32_t w[2][VB][2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int64_t bi = (c0 >> 5) + blk;
        const bool any = c0 + 32 * blk < t_end;
#pragma unroll
        for (int p = 0; p < VB; ++p) {
          if (any) {
            const uint2 x = *reinterpret_cast<const uint2*>(vp + (bi * VB + p) * kD + ch);
            w[blk][p][0] = x.x;
            w[blk][p][1] = x.y;
          } else {
            w[blk][p][0] = w[blk][p][1] = 0u;
          }
        }
      }
      const int grp = ch / a.value_group;
#pragma unroll 4
      for (int j = 0; j < kChunk; ++j) {
        const int blk = j >> 5, tb = j & 31;
        uint32_t w0[VB], w1[VB];
#pragma unroll
        for (int p = 0; p < VB; ++p) {
          w0[p] = w[blk][p][0];
          w1[p] = w[blk][p][1];
        }
        const uint32_t code0 = value_code<VB, packed_value_codes(VMSE, VB)>(w0, tb);
        const uint32_t code1 = value_code<VB, packed_value_codes(VMSE, VB)>(w1, tb);
        float v0, v1;
        if (VMSE) {
          const float nv = __uint_as_float(mb[wave][j][0]);
          v0 = nv * vc[code0];
          v1 = nv * vc[code1];
        } else {
          const uint32_t mm = mb[wave][j][grp];
          const float dlt = __half2float(__ushort_as_half((unsigned short)(mm & 0xffffu)));
          const float mn = __half2float(__ushort_as_half((unsigned short)(mm >> 16)));
          v0 = fmaf(dlt, (float)code0, mn);
          v1 = fmaf(dlt, (float)code1, mn);
        }
        const floatx4 p0 = *reinterpret_cast<const floatx4*>(&pb[wave][j][0]);
        const floatx4 p1 = *reinterpret_cast<const floatx4*>(&pb[wave][j][4]);
        acc0[0] = fmaf(p0[0], v0, acc0[0]);
        acc1[0] = fmaf(p0[0], v1, acc1[0]);
        acc0[1] = fmaf(p0[1], v0, acc0[1]);
        acc1[1] = fmaf(p0[1], v1, acc1[1]);
        acc0[2] = fmaf(p0[2], v0, acc0[2]);
        acc1[2] = fmaf(p0[2], v1, acc1[2]);
        acc0[3] = fmaf(p0[3], v0, acc0[3]);
        acc1[3] = fmaf(p0[3], v1, acc1[3]);
        if (G > 4) {
          acc0[4] = fmaf(p1[0], v0, acc0[4]);
          acc1[4] = fmaf(p1[0], v1, acc1[4]);
          acc0[5] = fmaf(p1[1], v0, acc0[5]);
          acc1[5] = fmaf(p1[1], v1, acc1[5]);
          acc0[6] = fmaf(p1[2], v0, acc0[6]);
          acc1[6] = fmaf(p1[2], v1, acc1[6]);
          acc0[7] = fmaf(p1[3], v0, acc0[7]);
          acc1[7] = fmaf(p1[3], v1, acc1[7]);
        }
      }
    }
    __syncthreads();  // pb/mb are rewritten by the next iteration
  }

  // ---- merge the four waves, write one partial (m, l, acc[128]) per query head
  __shared__ float macc[4][kMaxGroup][kD];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g >= G) break;
    const float l = wave_sum(l_part[g]);
    if (lane == 0) {
      mrg[wave][g][0] = m_run[g];
      mrg[wave][g][1] = l;
    }
    macc[wave][g][2 * lane] = acc0[g];
    macc[wave][g][2 * lane + 1] = acc1[g];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kD; i += blockDim.x) {
    const int g = i / kD, c = i % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg[w][g][0]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = mrg[w][g][0] == -INFINITY ? 0.f : __expf(mrg[w][g][0] - M);
        L += f * mrg[w][g][1];
        A += f * macc[w][g][c];
      }
    }
    float* part = a.partial + ((size_t)split * a.batch * a.h_kv * G + ws_row(a, b, h, g)) * (kD + 2);
    if (c == 0) {
      part[0] = M;
      part[1] = L;
    }
    part[2 + c] = A;
  }
}

// Combine as its own kernel: work-group of kCombineThreads per (sequence, KV
// head, virtual head).  Largest split count it stages in LDS (decode_split
// never splits a slot into more than kSplitTarget parts).
constexpr int kMaxCombineSplits = (int)kSplitTarget;

// Split accumulator words per thread loaded up front: 8 (a quarter of up to
// 32 splits) or, for slots split more than that, 24 (up to 96 splits, the
// long-sequence splits, in one round trip).
constexpr int kCombinePreShort = 8, kCombinePreLong = 24;

template <bool VMSE, int PRE>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(DecodeArgs a) {
  __shared__ CombineLds<kMaxCombineSplits> lds;
  const int rows = a.h_kv * a.group;
  const int b = blockIdx.x / rows, h = (blockIdx.x % rows) / a.group, gq = blockIdx.x % a.group;
  combine_unit<VMSE, kMaxCombineSplits, PRE>(a, b, h, gq, lds, a.partial + ws_row(a, b, h, gq) * (kD + 2),
                                        (size_t)a.batch * a.h_kv * a.group * (kD + 2));
}

__global__ void ring_append_kernel(const void* k_new, const void* v_new, int in_bf16, int h_kv,
                                   uint16_t* ring_k, uint16_t* ring_v, int ring_cap, SeqValues nr) {
  const int b = blockIdx.x / h_kv, h = blockIdx.x % h_kv, c = threadIdx.x;
  const size_t src = ((size_t)b * h_kv + h) * kD + c;
  const size_t dst = (((size_t)b * ring_cap + nr.v[b]) * h_kv + h) * kD + c;
  if (in_bf16) {
    ring_k[dst] = reinterpret_cast<const uint16_t*>(k_new)[src];
    ring_v[dst] = reinterpret_cast<const uint16_t*>(v_new)[src];
  } else {
    ring_k[dst] = (uint16_t)f2bf(reinterpret_cast<const float*>(k_new)[src]);
    ring_v[dst] = (uint16_t)f2bf(reinterpret_cast<const float*>(v_new)[src]);
  }
}

template <int KB, bool QJL, bool VMSE, int VB>
hipError_t launch_scan(const DecodeArgs& a, hipStream_t st, TimedLaunch tl) {
  launch_maybe_timed(scan_kernel<KB, QJL, VMSE, VB>, dim3(a.splits, a.batch * a.h_kv), dim3(kScanThreads), st, tl,
                     a);
  return hipGetLastError();
}

template <int KB, bool QJL, bool VMSE>
hipError_t dispatch_vb(const DecodeArgs& a, int vb, hipStream_t st, TimedLaunch tl) {
  switch (vb) {
    case 1: return launch_scan<KB, QJL, VMSE, 1>(a, st, tl);
    case 2: return launch_scan<KB, QJL, VMSE, 2>(a, st, tl);
    case 3: return launch_scan<KB, QJL, VMSE, 3>(a, st, tl);
    case 4: return launch_scan<KB, QJL, VMSE, 4>(a, st, tl);
  }
  return hipErrorInvalidValue;
}

template <int KB, bool QJL>
hipError_t dispatch_vk(const DecodeArgs& a, int vmse, int vb, hipStream_t st, TimedLaunch tl) {
  return vmse ? dispatch_vb<KB, QJL, true>(a, vb, st, tl) : dispatch_vb<KB, QJL, false>(a, vb, st, tl);
}

template <int KB>
hipError_t dispatch_qjl(const DecodeArgs& a, int qjl, int vmse, int vb, hipStream_t st, TimedLaunch tl) {
  return qjl ? dispatch_vk<KB, true>(a, vmse, vb, st, tl) : dispatch_vk<KB, false>(a, vmse, vb, st, tl);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int key_mse_bits, int key_qjl, int value_mse,
                         int value_bits, hipStream_t stream, TimedLaunch tl) {
  hipLaunchKernelGGL(qprep_kernel, dim3(a.batch * a.h_kv), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (key_mse_bits) {
    case 1: e = dispatch_qjl<1>(a, key_qjl, value_mse, value_bits, stream, tl); break;
    case 2: e = dispatch_qjl<2>(a, key_qjl, value_mse, value_bits, stream, tl); break;
    case 3: e = dispatch_qjl<3>(a, key_qjl, value_mse, value_bits, stream, tl); break;
    case 4: e = dispatch_qjl<4>(a, key_qjl, value_mse, value_bits, stream, tl); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_combine(a, value_mse, stream);
}

hipError_t launch_combine(const DecodeArgs& a, int value_mse, hipStream_t stream) {
  const dim3 grid(a.batch * a.h_kv * a.group), block(kCombineThreads);
  const bool many = a.splits > kCombineQuarters * kCombinePreShort;
  if (value_mse) {
    if (many)
      hipLaunchKernelGGL((combine_kernel<true, kCombinePreLong>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((combine_kernel<true, kCombinePreShort>), grid, block, 0, stream, a);
  } else {
    if (many)
      hipLaunchKernelGGL((combine_kernel<false, kCombinePreLong>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((combine_kernel<false, kCombinePreShort>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_ring_append(const void* k_new, const void* v_new, int in_bf16, int batch,
                              int h_kv, uint16_t* ring_k, uint16_t* ring_v, int ring_cap,
                              const SeqValues& n_ring, hipStream_t stream) {
  hipLaunchKernelGGL(ring_append_kernel, dim3(batch * h_kv), dim3(kD), 0, stream, k_new, v_new,
                     in_bf16, h_kv, ring_k, ring_v, ring_cap, n_ring);
  return hipGetLastError();
}

}  // namespace tq
