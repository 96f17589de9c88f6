// Encode kernels for gfx950: the rotation y = Pi u and the QJL projection of
// the residual run as bf16-split MFMA GEMMs (the only dense contractions of the
// method), the Lloyd-Max bucketing, residual and sign sketch run in registers,
// and the codes are written as bit planes.
//
// Method (page "TurboQuant — Random rotation trước khi quantize, 3-bit KV cache
// không mất accuracy", section "Ý tưởng cốt lõi"; TurboQuantProd of page
// "turboquant/audit_claims.py", AUDIT 3):
//   n = |k|, y = Pi k / n, idx_i = #{t : t < y_i}, r = y - c[idx] (the residual
//   in rotated space; |r| equals the residual norm in the original space),
//   sigma = sign(S r_orig) = sign(S Pi^T r).
//
// Precision: bf16 inputs are exact in bf16, so Pi k = Pi_hi k + Pi_lo k needs
// two MFMA passes (Pi split into bf16 hi + lo, error ~2^-17 |Pi|); fp32 inputs
// add a third pass with k split into hi + lo.  The residual is fp32, so the QJL
// GEMM uses three passes (S' hi/lo x r hi/lo, dropping lo x lo).  fp32
// accumulation throughout.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// LDS holds each bf16 matrix as 128 rows of 16 16-byte chunks; chunk c of row r
// sits in slot c ^ 8*((c >> 1) & 1) ^ (r & 15).  The MFMA operand reads (lane
// (g, tc) takes chunk 4ks + g of row 16rt + tc) then fall on distinct banks
// within every group of lanes the LDS serves together.
__host__ __device__ constexpr int lds_slot(int row, int chunk) {
  return (chunk ^ (8 * ((chunk >> 1) & 1))) ^ (row & 15);
}
constexpr int kEncThreads = 512;    // 8 waves (2 per SIMD); each wave encodes one 32-token tile at a time

// Derive the bf16 operands from Pi and S (fp32, row-major [128][128]).
__global__ void prepare_params_kernel(const float* __restrict__ pi, const float* __restrict__ s,
                                      uint16_t* __restrict__ out) {
  const int i = blockIdx.x;   // row
  const int k = threadIdx.x;  // column (contraction index for S')
  // Pi split
  const float p = pi[i * kD + k];
  const uint32_t hi = f2bf(p);
  const uint32_t lo = f2bf(p - bf2f(hi));
  out[kOffPiHi / 2 + i * kD + k] = (uint16_t)hi;
  out[kOffPiLo / 2 + i * kD + k] = (uint16_t)lo;
  // S' = S Pi^T in double, at the permuted column
  const int j = sp_column(k);
  double acc = 0.0;
  for (int m = 0; m < kD; ++m) acc += (double)s[i * kD + m] * (double)pi[j * kD + m];
  const float x = (float)acc;
  const uint32_t shi = f2bf(x);
  const uint32_t slo = f2bf((float)(acc - (double)bf2f(shi)));
  out[kOffSpHi / 2 + i * kD + k] = (uint16_t)shi;
  out[kOffSpLo / 2 + i * kD + k] = (uint16_t)slo;
  // fp32 transposes for the decode's query rotation
  float* ft = reinterpret_cast<float*>(out);
  ft[kOffPiT / 4 + k * kD + i] = p;
  ft[kOffST / 4 + k * kD + i] = s[i * kD + k];
}

// Map a tile index to (sequence, head, 32-token destination block).
__device__ __forceinline__ void tile_coords(const EncodeArgs& a, int tile, int& b, int& h,
                                            int64_t& blk) {
  b = 0;
  while (b + 1 < a.batch && tile >= a.tile_start.v[b + 1]) ++b;
  const int64_t pos = a.pos.v[b];
  const int64_t blk0 = pos >> 5;
  const int64_t nblk = ((pos + a.n_new + 31) >> 5) - blk0;
  const int64_t r = tile - a.tile_start.v[b];
  h = (int)(r / nblk);
  blk = blk0 + r % nblk;
}

// Lane LANE of w0 and of w1 replaced by the two halves of the wave-uniform
// 64-bit value m (a ballot), as a plain per-lane select: every lane compares
// its own index, so no instruction reads a scalar that a VALU compare has just
// written (the hazard an inline-asm v_writelane would need its own wait
// states for).
template <int LANE>
__device__ __forceinline__ void write_lane2(uint32_t& w0, uint32_t& w1, uint64_t m, int lane) {
  const bool mine = lane == LANE;
  w0 = mine ? (uint32_t)m : w0;
  w1 = mine ? (uint32_t)(m >> 32) : w1;
}

// f(std::integral_constant<int, I>{}) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Store one word of a value bit plane; words of partly covered blocks keep the
// bits of tokens this call does not write.
__device__ __forceinline__ void store_plane_word(uint32_t* p, uint32_t w, uint32_t vmask) {
  if (vmask == 0xffffffffu)
    *p = w;
  else
    *p = (*p & ~vmask) | (w & vmask);
}

// Two fp32 values rounded to bf16 (nearest even), packed low | high << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Sum over the four 16-lane rows of the wave (every lane gets the total),
// through the cross-row lane swaps (no LDS traffic).
__device__ __forceinline__ float row_sum4(float x) {
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(u[0]) + __uint_as_float(u[1]);
}

// Rotation-based encode: each wave encodes one 32-token tile at a time (two
// 16-token column tiles of the MFMA), eight waves of a work-group share the
// bf16 split matrices staged in LDS.
//   VALUE = false: TurboQuantProd keys (MSE_BITS-bit Lloyd-Max + QJL if QJL),
//                  token-major key planes, |k| and |r|.
//   VALUE = true : TurboQuant-MSE values, token-transposed value planes, |v|.
//   HALF         : keys of fractional width MSE_BITS + 1/2: the coordinates of
//                  the even row tiles (i mod 32 < 16) use the (MSE_BITS + 1)-bit
//                  table, and their extra bit goes to a half plane.
template <bool IN_BF16, int MSE_BITS, bool QJL, bool VALUE, bool HALF = false>
__global__ __launch_bounds__(kEncThreads) void encode_rot_kernel(EncodeArgs a) {
  static_assert(!(HALF && VALUE), "the half-bit layout is a key layout");
  constexpr int NMAT = QJL ? 4 : 2;
  constexpr int NP = MSE_BITS + (HALF ? 1 : 0) + (QJL ? 1 : 0);  // bit planes written per token
  constexpr int LV = 1 << MSE_BITS;
  constexpr int LVH = HALF ? 2 * LV : LV;  // levels of the half-bit coordinates
  __shared__ __attribute__((aligned(16))) uint16_t lds[NMAT][kD][kD];

  // Stage Pi_hi, Pi_lo (and S'_hi, S'_lo) once per work-group.
  for (int idx = threadIdx.x; idx < NMAT * kD * (kD / 8); idx += blockDim.x) {
    const int m = idx / (kD * kD / 8), rem = idx % (kD * kD / 8);
    const int row = rem / (kD / 8), c8 = rem % (kD / 8);
    *reinterpret_cast<u32x4*>(&lds[m][row][8 * lds_slot(row, c8)]) =
        *reinterpret_cast<const u32x4*>(a.derived + (size_t)m * kD * kD + row * kD + c8 * 8);
  }
  __syncthreads();

  float cent[LV], thr[LV - 1], cent_hi[LVH], thr_hi[LVH - 1];
#pragma unroll
  for (int k = 0; k < LV; ++k) cent[k] = VALUE ? a.v_cent[k] : a.k_cent[k];
#pragma unroll
  for (int k = 0; k < LV - 1; ++k) thr[k] = VALUE ? a.v_thr[k] : a.k_thr[k];
#pragma unroll
  for (int k = 0; k < LVH; ++k) cent_hi[k] = HALF ? a.k_cent_hi[k] : cent[k < LV ? k : 0];
#pragma unroll
  for (int k = 0; k < LVH - 1; ++k) thr_hi[k] = HALF ? a.k_thr_hi[k] : thr[k < LV - 1 ? k : 0];
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: tile indices, and the per-sequence lookups they
  // drive, stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int tc = lane & 15;  // token inside a 16-token column tile
  const int g = lane >> 4;   // lane group: coordinates 8g..8g+7 of each k-step
  const void* src = VALUE ? a.v : a.k;
  // slot of chunk 4ks + g of row 16rt + tc is lslot ^ 4ks (ks only touches bits 2, 3)
  const int lslot = lds_slot(tc, g);

  // Source row and destination position of column tc of column tile ct.
  // Value planes: column tc of tile ct holds the token whose bit position in
  // the plane word is 16ct + tc, so the ballots below land in place.
  auto tile_rows = [&](int tl, int64_t (&row)[2], int64_t (&dp)[2], bool (&ok)[2]) {
    int b, h;
    int64_t blk;
    tile_coords(a, tl, b, h, blk);
    const int64_t pos = a.pos.v[b];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      dp[ct] = blk * 32 + (VALUE ? vslot(16 * ct + tc) : 16 * ct + tc);
      const int64_t t = dp[ct] - pos;
      ok[ct] = t >= 0 && t < a.n_new;
      row[ct] = ((int64_t)b * a.n_new + (ok[ct] ? t : 0)) * a.h_kv + h;
    }
  };
  for (int tile = blockIdx.x * nwaves + wave; tile < a.num_tiles; tile += gridDim.x * nwaves) {
    int b, h;
    int64_t blk;
    tile_coords(a, tile, b, h, blk);
    const int64_t slot = (int64_t)b * a.h_kv + h;
    int64_t row[2], dpos[2];
    bool valid[2];
    tile_rows(tile, row, dpos, valid);

    // ---- the tile: two 16-token column tiles, 32 coordinates per lane
    u32x4 kin[2][4], klo[2][4];
    float ss[2] = {0.f, 0.f};
    if (IN_BF16) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          // Rows of columns outside the written range are clamped to a real
          // token: the load stays in bounds and holds finite values.  MFMA
          // output columns depend only on their own input column, and such
          // columns are never stored, so they need no masking.
          // (inputs are read once: non-temporal loads)
          kin[ct][ks] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
              reinterpret_cast<const uint16_t*>(src) + row[ct] * kD + 32 * ks + 8 * g));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(kin[ct][ks][e] << 16);
            const float hi = __uint_as_float(kin[ct][ks][e] & 0xffff0000u);
            ss[ct] = fmaf(lo, lo, ss[ct]);
            ss[ct] = fmaf(hi, hi, ss[ct]);
          }
    } else {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const floatx4* fp = reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(src) + row[ct] * kD +
                                                               32 * ks + 8 * g);
          // clamped row: in bounds, finite, never stored; read once (non-temporal)
          const floatx4 f0 = __builtin_nontemporal_load(fp), f1 = __builtin_nontemporal_load(fp + 1);
          const float f[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t hp = pack_bf16x2(f[2 * e], f[2 * e + 1]);
            kin[ct][ks][e] = hp;
            klo[ct][ks][e] = pack_bf16x2(f[2 * e] - __uint_as_float(hp << 16),
                                         f[2 * e + 1] - __uint_as_float(hp & 0xffff0000u));
            ss[ct] = fmaf(f[2 * e], f[2 * e], ss[ct]);
            ss[ct] = fmaf(f[2 * e + 1], f[2 * e + 1], ss[ct]);
          }
        }
      }
    }
    float nrm[2], inv[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const float s2 = row_sum4(ss[ct]);
      nrm[ct] = sqrtf(s2);
      // a zero vector gets y = -0: its sign bit puts every coordinate in the
      // lower cell of the middle threshold, as #{t < 0} does
      inv[ct] = nrm[ct] > 0.f ? 1.0f / nrm[ct] : -0.0f;
    }

    // ---- GEMM 1: Y = Pi K^T (row tile rt = coordinates 16rt..16rt+15); bucketing.
    // Plane bits are gathered lane-locally first: bit (rt&1)*4 + rr of lw[p][ct][rt/2]
    // is coordinate 16rt + 4g + rr of token 16ct + tc.
    uint32_t lw[NP][2][4];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int m = 0; m < 4; ++m) lw[p][ct][m] = 0u;
    u32x4 rhi[2][4], rlo[2][4];
    float gg[2] = {0.f, 0.f};
    uint32_t vw[VALUE ? NP : 1][2];  // value planes: words of channels lane and lane+64
#pragma unroll
    for (int p = 0; p < (VALUE ? NP : 1); ++p) vw[p][0] = vw[p][1] = 0u;

    // Software pipeline over the row tiles: step st issues the LDS reads and
    // MFMAs of row tile st next to the VALU epilogue of row tile st - 1 (they
    // are independent), so operand latency and matrix work hide behind it.
    auto gemm1 = [&](auto RT, floatx4 (&acc)[2]) __attribute__((always_inline)) {
      constexpr int rt = decltype(RT)::value;
      acc[0] = acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 ahi = *reinterpret_cast<const u32x4*>(&lds[0][16 * rt + tc][8 * (lslot ^ (4 * ks))]);
        const u32x4 alo = *reinterpret_cast<const u32x4*>(&lds[1][16 * rt + tc][8 * (lslot ^ (4 * ks))]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          acc[ct] = mfma_bf16(ahi, kin[ct][ks], acc[ct]);
          acc[ct] = mfma_bf16(alo, kin[ct][ks], acc[ct]);
          if (!IN_BF16) acc[ct] = mfma_bf16(ahi, klo[ct][ks], acc[ct]);
        }
      }
    };
    auto epilogue = [&](auto RT, const floatx4 (&acc)[2]) __attribute__((always_inline)) {
      constexpr int rt = decltype(RT)::value;
      // half-bit layout: the even row tiles (coordinates i mod 32 < 16) use
      // the table with one more bit
      constexpr bool HI = HALF && (rt % 2 == 0);
      constexpr int LVR = HI ? LVH : LV;
      constexpr int MBR = HI ? MSE_BITS + 1 : MSE_BITS;
      constexpr int NPOS = LVR / 2 - 1;  // positive thresholds of the symmetric table
      const float* cen = HI ? cent_hi : cent;
      const float* thp = HI ? thr_hi : thr;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float res[4];
        // sign words: bit p of the index is the inverted sign bit of t[rr][p]
        uint32_t t[4][MSE_BITS + 1];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float y = acc[ct][rr] * inv[ct];
          const uint32_t yb = __float_as_uint(y);
          const float ay = fabsf(y);
          // centroids pass through an empty asm: opaque scalars, so the select
          // chain is not folded into a per-lane table lookup in memory
          float cm = cen[LVR / 2];
          asm("" : "+s"(cm));
#pragma unroll
          for (int p = 0; p < MBR - 1; ++p) t[rr][p] = yb;
#pragma unroll
          for (int k = 1; k <= NPOS; ++k) {
            const float dk = ay - thp[LVR / 2 - 1 + k];
            float ck = cen[LVR / 2 + k];
            asm("" : "+s"(ck));
            cm = (int)__float_as_uint(dk) >= 0 ? ck : cm;  // the same sign bit as the index bits
#pragma unroll
            for (int p = 0; p < MBR - 1; ++p)
              if ((k & ((1 << p) - 1)) == 0) t[rr][p] ^= __float_as_uint(dk);
          }
          t[rr][MBR - 1] = yb;
          res[rr] = y - __uint_as_float(__float_as_uint(cm) | (yb & 0x80000000u));
          if (!VALUE) {
#pragma unroll
            for (int p = 0; p < MBR; ++p) {
              lw[p][ct][rt >> 1] = __builtin_amdgcn_alignbit(lw[p][ct][rt >> 1], t[rr][p], 31);
              // fold the bit in now, so the sign words of a row tile are not all kept live
              asm volatile("" : "+v"(lw[p][ct][rt >> 1]));
            }
          }
        }
        if (!VALUE && rt % 2 == 0) {
          // elements 0..3 of the word move up by 12: after the bit reversal
          // they sit 16 bits below elements 4..7
#pragma unroll
          for (int p = 0; p < MBR; ++p) lw[p][ct][rt >> 1] <<= 12;
        }
        if (HALF && !HI) lw[MSE_BITS][ct][rt >> 1] <<= 4;  // no half-plane bits in this tile
        if (QJL) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) gg[ct] = fmaf(res[rr], res[rr], gg[ct]);
          // element e = (rt&1)*4 + rr of the k-step rt/2 B operand of GEMM 2
#pragma unroll
          for (int hp = 0; hp < 2; ++hp) {
            const float r0 = res[2 * hp], r1 = res[2 * hp + 1];
            const uint32_t hi = pack_bf16x2(r0, r1);
            const uint32_t lo = pack_bf16x2(r0 - __uint_as_float(hi << 16), r1 - __uint_as_float(hi & 0xffff0000u));
            rhi[ct][rt >> 1][(rt & 1) * 2 + hp] = hi;
            rlo[ct][rt >> 1][(rt & 1) * 2 + hp] = lo;
          }
        }
        if (VALUE) {
          // token-transposed planes: one ballot gives, in bits 16g'..16g'+15, the
          // bit of channel 16rt + 4g' + rr for the 16 tokens of column tile ct
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const uint64_t m = __ballot((int)t[rr][p] >= 0);
#pragma unroll
              for (int gq = 0; gq < 4; ++gq) {
                const int ch = 16 * rt + 4 * gq + rr;
                const uint32_t w = (uint32_t)((m >> (16 * gq)) & 0xffffu) << (16 * ct);
                if (lane == (ch & 63)) vw[p][ch >> 6] |= w;
              }
            }
        }
      }
        };
    // (row tiles are compile-time constants, so every register array index is)
    floatx4 acc_c[2], acc_n[2];
    auto step = [&](auto ST) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value;
      // one step at a time: later row tiles' operands are not hoisted
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (st < 8) gemm1(std::integral_constant<int, st>{}, acc_n);
      if constexpr (st >= 1) epilogue(std::integral_constant<int, (st >= 1 ? st - 1 : 0)>{}, acc_c);
      acc_c[0] = acc_n[0];
      acc_c[1] = acc_n[1];
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 7>{});
    step(std::integral_constant<int, 8>{});

    if (VALUE) {
      // word bit 16ct + tc belongs to column tc of tile ct: valid-token mask
      const uint32_t vmask = (uint32_t)(__ballot(valid[0]) & 0xffffu) |
                             ((uint32_t)(__ballot(valid[1]) & 0xffffu) << 16);
      const int64_t nblk_cap = a.capacity >> 5;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        uint32_t* base = a.v_planes + ((slot * nblk_cap + blk) * NP + p) * kD;
        store_plane_word(base + lane, vw[p][0], vmask);
        store_plane_word(base + 64 + lane, vw[p][1], vmask);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        if (valid[ct] && g == 0) store_scalar(a.v_norm, slot * a.capacity + dpos[ct], nrm[ct], a.scalar_f16);
      continue;
    }

    float gam[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) gam[ct] = sqrtf(row_sum4(gg[ct]));

    // ---- GEMM 2: Z = S' R (QJL projection of the rotated residual), signs
    if (QJL) {
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        __builtin_amdgcn_sched_barrier(0);
        floatx4 z[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 ahi = *reinterpret_cast<const u32x4*>(&lds[2 % NMAT][16 * rt + tc][8 * (lslot ^ (4 * ks))]);
          const u32x4 alo = *reinterpret_cast<const u32x4*>(&lds[3 % NMAT][16 * rt + tc][8 * (lslot ^ (4 * ks))]);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            z[ct] = mfma_bf16(ahi, rhi[ct][ks], z[ct]);
            z[ct] = mfma_bf16(alo, rhi[ct][ks], z[ct]);
            z[ct] = mfma_bf16(ahi, rlo[ct][ks], z[ct]);
          }
        }
        // shift the sign bit of z in at the bottom, with the gap of 12 after
        // the even row tile (the bit layout of the plane words below)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            lw[NP - 1][ct][rt >> 1] = __builtin_amdgcn_alignbit(lw[NP - 1][ct][rt >> 1], __float_as_uint(z[ct][rr]), 31);
        if (rt % 2 == 0) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) lw[NP - 1][ct][rt >> 1] <<= 12;
        }
      }
    }
    // ---- plane words.  Every plane bit went in as a sign bit shifted in at
    // the bottom, with a gap of 12 after element 3 of a word (element j =
    // (rt&1)*4 + rr of word rt/2): bit reversal puts element j at bit 12 + j
    // (j < 4) or 24 + j.  Inverted, bit j is 1 where the sign word was
    // non-negative.  The Lloyd-Max index bits are the sign of y (top bit) and
    // the parity of the magnitude tests against the positive thresholds XOR
    // that sign (lower bits); each of them has an odd number of tests, hence
    // the inversion.  Ties (|y| on a threshold, y = 0, z = -0.0) lie inside
    // the boundary window of the oracle's values.  A shift then spreads the
    // bits to coordinate positions 4g + j (j < 4) and 16 + 4g + j - 4, and the
    // lane swaps gather the word of coordinates 32g..32g+31 into lane group g.
    // record: full planes at 16p, the half plane (16 coordinates per lane
    // group) at 16 MSE_BITS, the QJL plane after it
    constexpr size_t rec = (size_t)(MSE_BITS + (QJL ? 1 : 0)) * (kD / 8) + (HALF ? kD / 16 : 0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) w[m] = (~__builtin_bitreverse32(lw[p][ct][m]) >> (12 - 4 * g)) & (0x000f000fu << (4 * g));
        // lanes g and g^2 merge: rows 0,1 keep words 0,1 and rows 2,3 words 2,3
        const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        const uint32_t ka = s02[0] | s02[1], kb = s13[0] | s13[1];
        // then rows g and g^1: row g ends with word g
        const auto sf = __builtin_amdgcn_permlane16_swap(ka, kb, false, false);
        const uint32_t fin = sf[0] | sf[1];
        uint8_t* kslot = a.k_planes + slot * key_slot_tokens(a.capacity) * rec;
        if (valid[ct]) {
          if (HALF && p == MSE_BITS)  // coordinates 32g..32g+15: the low half of the word
            *reinterpret_cast<uint16_t*>(kslot + key_word_offset(dpos[ct], rec, MSE_BITS * (kD / 8), g, 2)) =
                (uint16_t)fin;
          else
            *reinterpret_cast<uint32_t*>(
                kslot + key_word_offset(dpos[ct], rec,
                                        p < MSE_BITS ? p * (kD / 8) : MSE_BITS * (kD / 8) + (HALF ? kD / 16 : 0), g,
                                        4)) = fin;
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      if (valid[ct] && g == 0) {
        store_scalar(a.k_norm, slot * a.capacity + dpos[ct], nrm[ct], a.scalar_f16);
        if (QJL) store_scalar(a.k_rnorm, slot * a.capacity + dpos[ct], gam[ct], a.scalar_f16);
      }
    }
  }
}

// Bit position, in a 32-token value-plane word, of the token at position u of
// its block (the inverse of vslot).
__device__ __forceinline__ int vslot_inv(int u) { return 8 * (u & 3) + 4 * (u >> 4) + ((u >> 2) & 3); }

// Sum over the 128 threads of a work-group (two waves), every thread gets it.
__device__ __forceinline__ float block_sum128(float x, float* red) {
  x = wave_sum(x);
  __syncthreads();  // red is free again
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return red[0] + red[1];
}

// Column i of a 128 x 128 fp32 matrix M (row-major, M[k][i] at k * kD + i),
// read into registers with every load issued before any is used (one memory
// round trip instead of one per group of unrolled loads), and its product with
// the staged vector xs: sum_k M[k][i] xs[k].
struct Col128 {
  float m[kD];
};
__device__ __forceinline__ Col128 load_col128(const float* M, int i) {
  // the matrix does not change inside the token loop, but its column is read
  // per token: an opaque copy of the pointer keeps the loads where they are
  // written, so one column at a time is live
  asm volatile("" : "+s"(M));
  Col128 c;
#pragma unroll
  for (int k = 0; k < kD; ++k) c.m[k] = M[k * kD + i];
  return c;
}
__device__ __forceinline__ float col_dot128(const Col128& c, const float* xs) {
  asm volatile("" ::: "memory");  // the column's loads are all issued before the products start
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kD; ++k) acc = fmaf(c.m[k], xs[k], acc);
  asm volatile("" ::: "memory");  // and no later column's loads start before they end (one column live)
  return acc;
}

// Few-token encode (a decode step's new tokens): one work-group of 128
// threads per (sequence, head, 32-token block) tile, one thread per
// coordinate, in fp32 with coalesced column reads of fp32 matrices.  Per
// token: n = |k|, y = Pi k / n (Pi^T from the derived buffer), the Lloyd-Max
// index #{t < y_i} with the coordinate's own table, and for QJL keys the
// residual in the original space r = Pi^T (y - c) (Pi from the caller's
// parameters), z = S r (S^T from the derived buffer), gamma = |y - c|.  No
// LDS staging of the matrices: for a handful of tokens that staging would
// cost more than the products.
template <bool IN_BF16, int MSE_BITS, bool QJL, bool VALUE, bool HALF>
__device__ __forceinline__ void encode_small_body(EncodeArgs a) {
  static_assert(!(HALF && VALUE), "the half-bit layout is a key layout");
  constexpr int LV = 1 << MSE_BITS;
  __shared__ float xs[kD];
  __shared__ float red[2];
  const int i = threadIdx.x, lane = i & 63, wv = i >> 6;
  int b, h;
  int64_t blk;
  tile_coords(a, blockIdx.x, b, h, blk);
  const int64_t pos = a.pos.v[b];
  const int64_t slot = (int64_t)b * a.h_kv + h;
  const float* pit = reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.derived) + kOffPiT);
  const float* stt = reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.derived) + kOffST);
  const void* src = VALUE ? a.v : a.k;
  const bool hi = HALF && (i & 31) < 16;  // this coordinate uses the table with one more bit
  constexpr size_t rec = (size_t)(MSE_BITS + (QJL ? 1 : 0)) * (kD / 8) + (HALF ? kD / 16 : 0);
  uint32_t vw[MSE_BITS];  // value planes: this channel's word of each plane for the block
#pragma unroll
  for (int p = 0; p < MSE_BITS; ++p) vw[p] = 0u;
  uint32_t vmask = 0u;
  for (int u = 0; u < 32; ++u) {
    const int64_t dp = blk * 32 + u;
    const int64_t t = dp - pos;
    if (t < 0 || t >= a.n_new) continue;  // the same for every thread
    const int64_t row = ((int64_t)b * a.n_new + t) * a.h_kv + h;
    const float x = IN_BF16 ? bf2f(reinterpret_cast<const uint16_t*>(src)[row * kD + i])
                            : reinterpret_cast<const float*>(src)[row * kD + i];
    const Col128 cpi = load_col128(pit, i);  // in flight with the token's own load and norm
    const float n = sqrtf(block_sum128(x * x, red));
    const float inv = n > 0.f ? 1.0f / n : 0.f;
    xs[i] = x;
    __syncthreads();
    const float y = col_dot128(cpi, xs) * inv;
    int idx = 0;
    float c;
    if (hi) {
#pragma unroll
      for (int k = 0; k < 2 * LV - 1; ++k) idx += y > a.k_thr_hi[k] ? 1 : 0;
      c = a.k_cent_hi[idx];
    } else {
      const float* thr = VALUE ? a.v_thr : a.k_thr;
#pragma unroll
      for (int k = 0; k < LV - 1; ++k) idx += y > thr[k] ? 1 : 0;
      c = VALUE ? a.v_cent[idx] : a.k_cent[idx];
    }
    if (VALUE) {
      const int bp = vslot_inv(u);
#pragma unroll
      for (int p = 0; p < MSE_BITS; ++p) vw[p] |= (uint32_t)((idx >> p) & 1) << bp;
      vmask |= 1u << bp;
      if (i == 0) store_scalar(a.v_norm, slot * a.capacity + dp, n, a.scalar_f16);
      __syncthreads();  // xs is rewritten by the next token
      continue;
    }
    const float r = y - c;
    bool zbit = false;
    float gam = 0.f;
    if (QJL) {
      const Col128 cp = load_col128(a.pi, i);  // (Pi^T r)_i = sum_j Pi[j][i] r_j
      gam = sqrtf(block_sum128(r * r, red));  // its barriers also end the reads of xs
      xs[i] = r;
      __syncthreads();
      const float ro = col_dot128(cp, xs);
      const Col128 cs = load_col128(stt, i);  // (S ro)_i = sum_j S^T[j][i] ro_j
      __syncthreads();
      xs[i] = ro;
      __syncthreads();
      zbit = col_dot128(cs, xs) >= 0.f;
    }
    // plane words by ballot: wave wv holds coordinates 64 wv .. 64 wv + 63,
    // the words 2 wv and 2 wv + 1 of every plane
    uint8_t* kslot = a.k_planes + slot * key_slot_tokens(a.capacity) * rec;
#pragma unroll
    for (int p = 0; p < MSE_BITS; ++p) {
      const uint64_t m = __ballot((idx >> p) & 1);
      if (lane == 0) {
        *reinterpret_cast<uint32_t*>(kslot + key_word_offset(dp, rec, p * (kD / 8), 2 * wv, 4)) = (uint32_t)m;
        *reinterpret_cast<uint32_t*>(kslot + key_word_offset(dp, rec, p * (kD / 8), 2 * wv + 1, 4)) = (uint32_t)(m >> 32);
      }
    }
    if (HALF) {  // the extra bit of the half-bit coordinates: the low 16 bits of each word
      const uint64_t m = __ballot(hi && ((idx >> MSE_BITS) & 1));
      if (lane == 0) {
        *reinterpret_cast<uint16_t*>(kslot + key_word_offset(dp, rec, MSE_BITS * (kD / 8), 2 * wv, 2)) =
            (uint16_t)(m & 0xffffu);
        *reinterpret_cast<uint16_t*>(kslot + key_word_offset(dp, rec, MSE_BITS * (kD / 8), 2 * wv + 1, 2)) =
            (uint16_t)((m >> 32) & 0xffffu);
      }
    }
    if (QJL) {
      const uint64_t m = __ballot(zbit);
      const int off = MSE_BITS * (kD / 8) + (HALF ? kD / 16 : 0);
      if (lane == 0) {
        *reinterpret_cast<uint32_t*>(kslot + key_word_offset(dp, rec, off, 2 * wv, 4)) = (uint32_t)m;
        *reinterpret_cast<uint32_t*>(kslot + key_word_offset(dp, rec, off, 2 * wv + 1, 4)) = (uint32_t)(m >> 32);
      }
    }
    if (i == 0) {
      store_scalar(a.k_norm, slot * a.capacity + dp, n, a.scalar_f16);
      if (QJL) store_scalar(a.k_rnorm, slot * a.capacity + dp, gam, a.scalar_f16);
    }
    __syncthreads();  // xs is rewritten by the next token
  }
  if (VALUE && vmask) {
    const int64_t nblk_cap = a.capacity >> 5;
#pragma unroll
    for (int p = 0; p < MSE_BITS; ++p)
      store_plane_word(a.v_planes + ((slot * nblk_cap + blk) * MSE_BITS + p) * kD + i, vw[p], vmask);
  }
}

template <bool IN_BF16, int MSE_BITS, bool QJL, bool VALUE, bool HALF>
__global__ __launch_bounds__(kD) void encode_small_kernel(EncodeArgs a) {
  encode_small_body<IN_BF16, MSE_BITS, QJL, VALUE, HALF>(a);
}

// Keys (QJL) and MSE values of the same few tokens in one launch: the two
// codes share no data, so work-groups (tile, 0) encode the keys and (tile, 1)
// the values, and the two run side by side instead of one after the other.
template <bool IN_BF16, int KEY_BITS, int VAL_BITS>
__global__ __launch_bounds__(kD) void encode_small_kv_kernel(EncodeArgs a) {
  if (blockIdx.y == 0)
    encode_small_body<IN_BF16, KEY_BITS, true, false, false>(a);
  else
    encode_small_body<IN_BF16, VAL_BITS, false, true, false>(a);
}

// DPP move of a 32-bit value (all lanes active).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xf, 0xf, false);
}

// Bit offset of token i (0..15) in a packed 2-bit code word.
__device__ __forceinline__ constexpr int packed2_offset(int i) { return 8 * (i & 3) + 2 * (i >> 2); }

// 16 x 16 transpose of 2-bit fields inside each 16-lane row: on entry lane i
// of the row holds in D[m] the fields (i, j) at packed2_offset(j); on exit
// lane j holds the fields (i, j) at packed2_offset(i).  Stage k swaps lane
// index bit k with field index bit k (field stride S_k): each lane keeps the
// fields whose index bit k equals its own lane bit k and takes the others
// from lane i ^ 2^k, rotated by S_k.  The partners come from quad
// permutations, a half-row mirror then a quad reversal (lane i ^ 4), and a
// rotation by 8 (lane i ^ 8); all four are their own inverses.
__device__ __forceinline__ void transpose16_2bit(uint32_t (&D)[4], int li) {
  constexpr uint32_t kM0[4] = {0x00ff00ffu, 0x0000ffffu, 0x33333333u, 0x0f0f0f0fu};
  constexpr int kS[4] = {8, 16, 2, 4};
  static_for<0, 4>([&](auto K) {
    constexpr int k = decltype(K)::value;
    const bool ak = (li >> k) & 1;
    const uint32_t keep = ak ? (kM0[k] << kS[k]) : kM0[k];
    const int sh = ak ? kS[k] : 32 - kS[k];  // rotate right by sh
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t P;
      if constexpr (k == 0) P = dpp_u32<0xb1>(D[m]);                 // quad_perm [1, 0, 3, 2]
      else if constexpr (k == 1) P = dpp_u32<0x4e>(D[m]);            // quad_perm [2, 3, 0, 1]
      else if constexpr (k == 2) P = dpp_u32<0x1b>(dpp_u32<0x141>(D[m]));  // half-row mirror, quad reversal
      else P = dpp_u32<0x128>(D[m]);                                 // row rotation by 8
      const uint32_t rot = __builtin_amdgcn_alignbit(P, P, sh);
      D[m] = (D[m] & keep) | (rot & ~keep);
    }
  });
}

// Bit offset of token i (0..7) in a packed 4-bit code word.
__device__ __forceinline__ constexpr int packed4_offset(int i) { return 8 * (i & 3) + 4 * (i >> 2); }

// The same transpose for 4-bit fields, 8 x 8 inside each 8-lane half-row
// (three stages: lane i ^ 1, i ^ 2, i ^ 4).
__device__ __forceinline__ void transpose8_4bit(uint32_t (&D)[8], int li) {
  constexpr uint32_t kM0[3] = {0x00ff00ffu, 0x0000ffffu, 0x0f0f0f0fu};
  constexpr int kS[3] = {8, 16, 4};
  static_for<0, 3>([&](auto K) {
    constexpr int k = decltype(K)::value;
    const bool ak = (li >> k) & 1;
    const uint32_t keep = ak ? (kM0[k] << kS[k]) : kM0[k];
    const int sh = ak ? kS[k] : 32 - kS[k];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t P;
      if constexpr (k == 0) P = dpp_u32<0xb1>(D[m]);
      else if constexpr (k == 1) P = dpp_u32<0x4e>(D[m]);
      else P = dpp_u32<0x1b>(dpp_u32<0x141>(D[m]));
      const uint32_t rot = __builtin_amdgcn_alignbit(P, P, sh);
      D[m] = (D[m] & keep) | (rot & ~keep);
    }
  });
}

// Asymmetric min/max value code, one 32-token tile per wave: lane = (token,
// half of the channels).  The stored scale and zero are exact functions of the
// group (correctly rounded fp32 division, then fp16):
//   delta = fp16(fp32(max - min) / (2^b - 1)), zero = fp16(min)
//   code  = clamp(rint(fp32(v - zero) * fp32(1 / delta)), 0, 2^b - 1), 0 if delta == 0
// in IEEE fp32 with every step correctly rounded.  The rounding to an integer
// (ties to even) is the addition of 1.5 * 2^23, which leaves the code, biased by
// that number's bit pattern, in the low bits of the sum; an integer clamp to
// [bias, bias + 2^b - 1] then saturates quotients outside the code range, of
// any size and sign.  A quotient that is exactly a midpoint k + 1/2 in fp32 (it
// happens: the inputs are bf16 or fp16 numbers) rounds to even, as the plain
// definition does.
constexpr float kRoundBias = 12582912.0f;  // 1.5 * 2^23: adding it rounds to an integer
constexpr int kBiasBits = 0x4B400000;       // its bit pattern, the code 0 after the addition

// Sum over the fields of a packed word (field j at bit 8 (j % 4) + W (j / 4),
// N fields of width W) of the bias each biased code carries, modulo 2^32:
// subtracting it from the sum of the shifted biased codes leaves the codes,
// since their fields do not overlap.
template <int N, int W>
constexpr uint32_t packed_bias() {
  uint32_t c = 0u;
  for (int j = 0; j < N; ++j) c += (uint32_t)kBiasBits << (8 * (j & 3) + W * (j >> 2));
  return c;
}

template <bool IN_BF16, int BITS, int GS>
__global__ __launch_bounds__(256) void encode_minmax_kernel(EncodeArgs a) {
  constexpr int L = (1 << BITS) - 1;
  constexpr int NG = 64 / GS;  // groups per lane
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: tile indices, and the per-sequence lookups they
  // drive, stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  // lane l (mod 32) encodes the token whose bit position in a plane word is
  // l mod 32, so a ballot over the wave is already the plane word
  // (2- and 4-bit codes: token = lane % 32 in order, and each 16-lane row or
  // 8-lane half-row builds its packed words by an in-register transpose)
  const int tok = (BITS == 2 || BITS == 4) ? (lane & 31) : vslot(lane & 31), half = lane >> 5;
  for (int tile = blockIdx.x * nwaves + wave; tile < a.num_tiles; tile += gridDim.x * nwaves) {
    int b, h;
    int64_t blk;
    tile_coords(a, tile, b, h, blk);
    const int64_t pos = a.pos.v[b];
    const int64_t slot = (int64_t)b * a.h_kv + h;
    const int64_t dp = blk * 32 + tok;
    const int64_t t = dp - pos;
    const bool valid = t >= 0 && t < a.n_new;
    // the row of a token outside the written range is clamped to a real one:
    // the load stays in bounds, and neither its codes nor its scales are stored
    const int64_t row = ((int64_t)b * a.n_new + (valid ? t : 0)) * a.h_kv + h;
    float x[64];
    if (IN_BF16) {
      const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.v) + row * kD + 64 * half);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 w = p[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * i + 2 * e] = bf2f(w[e] & 0xffffu);
          x[8 * i + 2 * e + 1] = bf2f(w[e] >> 16);
        }
      }
    } else {
      const floatx4* p = reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(a.v) + row * kD + 64 * half);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const floatx4 w = p[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * i + e] = w[e];
      }
    }
    uint32_t code[64];
    const int ngroups_row = kD / GS;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float mn = x[gi * GS], mx = x[gi * GS];
#pragma unroll
      for (int e = 1; e < GS; ++e) {
        mn = fminf(mn, x[gi * GS + e]);
        mx = fmaxf(mx, x[gi * GS + e]);
      }
      const __half d16 = __float2half_rn(__fdiv_rn(__fsub_rn(mx, mn), (float)L));
      const __half z16 = __float2half_rn(mn);
      const float d32 = __half2float(d16), z32 = __half2float(z16);
      // delta == 0 (a constant group): a zero factor leaves every code at 0
      const float invd = d32 != 0.f ? __fdiv_rn(1.0f, d32) : 0.f;
#pragma unroll
      for (int e = 0; e < GS; ++e) {
        // the product is rounded before the addition (no fused multiply-add)
#pragma clang fp contract(off)
        const float q = (x[gi * GS + e] - z32) * invd;
        const float f = q + kRoundBias;
        code[gi * GS + e] = (uint32_t)min(max(__float_as_int(f), kBiasBits), kBiasBits + L);  // biased code
      }
      if (valid) {
        const int grp = half * NG + gi;
        uint16_t* m = a.v_meta + ((slot * a.capacity + dp) * ngroups_row + grp) * 2;
        const uint32_t packed = (uint32_t)__half_as_ushort(d16) | ((uint32_t)__half_as_ushort(z16) << 16);
        *reinterpret_cast<uint32_t*>(m) = packed;
      }
    }
    const int64_t nblk_cap = a.capacity >> 5;
    if constexpr (BITS == 2) {
      // lane (half, h, i) holds token 16 h + i: its 64 codes go to D[m] with
      // channel 16 m + j at the packed offset of token j, and the row
      // transpose leaves channel 64 half + 16 m + i of word h in D[m]
      const int li = lane & 15, hw = (lane >> 4) & 1;
      constexpr uint32_t kBias = packed_bias<16, 2>();
      uint32_t D[4] = {0u, 0u, 0u, 0u};
      static_for<0, 64>([&](auto E) {
        constexpr int e = decltype(E)::value;
        D[e >> 4] += code[e] << packed2_offset(e & 15);
      });
#pragma unroll
      for (int m = 0; m < 4; ++m) D[m] -= kBias;
      transpose16_2bit(D, li);
      // the word's valid tokens: OR of the row's own fields
      uint32_t msk = valid ? 3u << packed2_offset(li) : 0u;
      msk |= dpp_u32<0xb1>(msk);
      msk |= dpp_u32<0x4e>(msk);
      msk |= dpp_u32<0x124>(msk);
      msk |= dpp_u32<0x128>(msk);
      uint32_t* base = a.v_planes + ((slot * nblk_cap + blk) * BITS + hw) * kD + 64 * half + li;
#pragma unroll
      for (int m = 0; m < 4; ++m) store_plane_word(base + 16 * m, D[m], msk);
    } else if constexpr (BITS == 4) {
      // lane (half, h, i) holds token 8 h + i: channel 8 m + j at the packed
      // offset of token j in D[m]; the half-row transpose leaves channel
      // 64 half + 8 m + i of word h in D[m]
      const int li = lane & 7, hw = (lane >> 3) & 3;
      constexpr uint32_t kBias = packed_bias<8, 4>();
      uint32_t D[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      static_for<0, 64>([&](auto E) {
        constexpr int e = decltype(E)::value;
        D[e >> 3] += code[e] << packed4_offset(e & 7);
      });
#pragma unroll
      for (int m = 0; m < 8; ++m) D[m] -= kBias;
      transpose8_4bit(D, li);
      uint32_t msk = valid ? 15u << packed4_offset(li) : 0u;
      msk |= dpp_u32<0xb1>(msk);
      msk |= dpp_u32<0x4e>(msk);
      msk |= dpp_u32<0x1b>(dpp_u32<0x141>(msk));
      uint32_t* base = a.v_planes + ((slot * nblk_cap + blk) * BITS + hw) * kD + 64 * half + li;
#pragma unroll
      for (int m = 0; m < 8; ++m) store_plane_word(base + 8 * m, D[m], msk);
    } else {
      // token-transposed planes: ballot over the wave gives tokens 0..31 of
      // channel e (low half) and of channel 64 + e (high half)
      uint32_t w[BITS][2];
#pragma unroll
      for (int p = 0; p < BITS; ++p) w[p][0] = w[p][1] = 0u;
#pragma unroll
      for (int e = 0; e < 64; ++e) code[e] -= (uint32_t)kBiasBits;
      static_for<0, 64>([&](auto E) {
        constexpr int e = decltype(E)::value;
#pragma unroll
        for (int p = 0; p < BITS; ++p) {
          const uint64_t m = __ballot((code[e] >> p) & 1u);
          // the ballot is wave-uniform: write its halves straight into lane e
          write_lane2<e>(w[p][0], w[p][1], m, lane);
        }
      });
      const uint32_t vmask = (uint32_t)__ballot(valid);  // bit l: lane l's token is written
      uint32_t out[BITS][2], msk[BITS];
      if constexpr (packed_value_codes(false, BITS)) {
        // widths 2 and 4 are stored as packed codes
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          uint32_t pl[BITS], pk[BITS];
#pragma unroll
          for (int p = 0; p < BITS; ++p) pl[p] = w[p][hf];
          planes_to_packed<BITS>(pl, pk);
#pragma unroll
          for (int p = 0; p < BITS; ++p) out[p][hf] = pk[p];
        }
        mask_to_packed<BITS>(vmask, msk);
      } else {
#pragma unroll
        for (int p = 0; p < BITS; ++p) {
          out[p][0] = w[p][0];
          out[p][1] = w[p][1];
          msk[p] = vmask;
        }
      }
#pragma unroll
      for (int p = 0; p < BITS; ++p) {
        uint32_t* base = a.v_planes + ((slot * nblk_cap + blk) * BITS + p) * kD;
        store_plane_word(base + lane, out[p][0], msk[p]);
        store_plane_word(base + 64 + lane, out[p][1], msk[p]);
      }
    }
  }
}

int encode_grid(int tiles, int waves_per_block) {
  const int want = (tiles + waves_per_block - 1) / waves_per_block;
  return want < 1 ? 1 : want;
}

template <bool BF16, int MB, bool QJL, bool VALUE, bool HALF = false>
hipError_t launch_rot(const EncodeArgs& a, hipStream_t st, TimedLaunch tl) {
  int grid = encode_grid(a.num_tiles, kEncThreads / 64);
  const int cus = device_cu_count();
  if (grid > cus) grid = cus;  // persistent: the LDS staging is paid once per work-group
  if (tl.begin) (void)hipEventRecord(tl.begin, st);
  hipLaunchKernelGGL((encode_rot_kernel<BF16, MB, QJL, VALUE, HALF>), dim3(grid), dim3(kEncThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (tl.end) (void)hipEventRecord(tl.end, st);
  return e;
}

// Calls with at most this many new tokens per sequence take the few-token
// encode (TQ_ENCODE_PATH=small or =mfma forces one path).
constexpr int64_t kSmallEncodeTokens = 4;

bool use_small_encode(const EncodeArgs& a) {
  const char* path = std::getenv("TQ_ENCODE_PATH");
  if (path && std::strcmp(path, "small") == 0) return true;
  if (path && std::strcmp(path, "mfma") == 0) return false;
  return a.n_new <= kSmallEncodeTokens;
}

template <bool BF16, int MB, bool QJL, bool VALUE, bool HALF = false>
hipError_t launch_enc(const EncodeArgs& a, hipStream_t st, TimedLaunch tl) {
  if (!use_small_encode(a)) return launch_rot<BF16, MB, QJL, VALUE, HALF>(a, st, tl);
  if (tl.begin) (void)hipEventRecord(tl.begin, st);
  hipLaunchKernelGGL((encode_small_kernel<BF16, MB, QJL, VALUE, HALF>), dim3(a.num_tiles), dim3(kD), 0, st, a);
  hipError_t e = hipGetLastError();
  if (tl.end) (void)hipEventRecord(tl.end, st);
  return e;
}

template <bool BF16, bool QJL, bool VALUE>
hipError_t dispatch_rot_bits(const EncodeArgs& a, int bits, hipStream_t st, TimedLaunch tl) {
  switch (bits) {
    case 1: return launch_enc<BF16, 1, QJL, VALUE>(a, st, tl);
    case 2: return launch_enc<BF16, 2, QJL, VALUE>(a, st, tl);
    case 3: return launch_enc<BF16, 3, QJL, VALUE>(a, st, tl);
    case 4: return launch_enc<BF16, 4, QJL, VALUE>(a, st, tl);
  }
  return hipErrorInvalidValue;
}

template <bool BF16, int BITS>
hipError_t launch_mm(const EncodeArgs& a, hipStream_t st, TimedLaunch tl) {
  const int grid = encode_grid(a.num_tiles, 4);
  if (tl.begin) (void)hipEventRecord(tl.begin, st);
  switch (a.value_group) {
    case 16: hipLaunchKernelGGL((encode_minmax_kernel<BF16, BITS, 16>), dim3(grid), dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((encode_minmax_kernel<BF16, BITS, 32>), dim3(grid), dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((encode_minmax_kernel<BF16, BITS, 64>), dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (tl.end) (void)hipEventRecord(tl.end, st);
  return e;
}

template <bool BF16>
hipError_t dispatch_mm(const EncodeArgs& a, int bits, hipStream_t st, TimedLaunch tl) {
  switch (bits) {
    case 1: return launch_mm<BF16, 1>(a, st, tl);
    case 2: return launch_mm<BF16, 2>(a, st, tl);
    case 3: return launch_mm<BF16, 3>(a, st, tl);
    case 4: return launch_mm<BF16, 4>(a, st, tl);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prepare_params(const float* pi, const float* s, uint16_t* derived,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(prepare_params_kernel, dim3(kD), dim3(kD), 0, stream, pi, s, derived);
  return hipGetLastError();
}

hipError_t launch_encode_keys(const EncodeArgs& a, int in_bf16, int mse_bits, int qjl, int half,
                              hipStream_t stream, TimedLaunch tl) {
  if (a.num_tiles == 0) return hipSuccess;
  if (half) {  // fractional widths 1.5 and 2.5 MSE bits, QJL keys only
    if (!qjl || mse_bits < 1 || mse_bits > 2) return hipErrorInvalidValue;
    if (in_bf16)
      return mse_bits == 1 ? launch_enc<true, 1, true, false, true>(a, stream, tl)
                           : launch_enc<true, 2, true, false, true>(a, stream, tl);
    return mse_bits == 1 ? launch_enc<false, 1, true, false, true>(a, stream, tl)
                         : launch_enc<false, 2, true, false, true>(a, stream, tl);
  }
  if (in_bf16)
    return qjl ? dispatch_rot_bits<true, true, false>(a, mse_bits, stream, tl)
               : dispatch_rot_bits<true, false, false>(a, mse_bits, stream, tl);
  return qjl ? dispatch_rot_bits<false, true, false>(a, mse_bits, stream, tl)
             : dispatch_rot_bits<false, false, false>(a, mse_bits, stream, tl);
}

hipError_t launch_encode_small_kv(const EncodeArgs& a, int in_bf16, int key_mse_bits, int key_qjl, int key_half,
                                  int value_bits, hipStream_t stream) {
  if (a.num_tiles == 0) return hipSuccess;
  if (!use_small_encode(a) || !key_qjl || key_half || key_mse_bits < 2 || key_mse_bits > 3 || value_bits < 2 ||
      value_bits > 3)
    return hipErrorNotSupported;
  const dim3 grid(a.num_tiles, 2);
  const int sel = (in_bf16 ? 4 : 0) + (key_mse_bits == 3 ? 2 : 0) + (value_bits == 3 ? 1 : 0);
  switch (sel) {
    case 0: hipLaunchKernelGGL((encode_small_kv_kernel<false, 2, 2>), grid, dim3(kD), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((encode_small_kv_kernel<false, 2, 3>), grid, dim3(kD), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((encode_small_kv_kernel<false, 3, 2>), grid, dim3(kD), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((encode_small_kv_kernel<false, 3, 3>), grid, dim3(kD), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((encode_small_kv_kernel<true, 2, 2>), grid, dim3(kD), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((encode_small_kv_kernel<true, 2, 3>), grid, dim3(kD), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((encode_small_kv_kernel<true, 3, 2>), grid, dim3(kD), 0, stream, a); break;
    default: hipLaunchKernelGGL((encode_small_kv_kernel<true, 3, 3>), grid, dim3(kD), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_encode_values_mse(const EncodeArgs& a, int in_bf16, int bits, hipStream_t stream,
                                    TimedLaunch tl) {
  if (a.num_tiles == 0) return hipSuccess;
  return in_bf16 ? dispatch_rot_bits<true, false, true>(a, bits, stream, tl)
                 : dispatch_rot_bits<false, false, true>(a, bits, stream, tl);
}

hipError_t launch_encode_values_minmax(const EncodeArgs& a, int in_bf16, int bits,
                                       hipStream_t stream, TimedLaunch tl) {
  if (a.num_tiles == 0) return hipSuccess;
  return in_bf16 ? dispatch_mm<true>(a, bits, stream, tl) : dispatch_mm<false>(a, bits, stream, tl);
}

}  // namespace tq
