// Device helpers shared by the encode and decode kernels.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Bit position, inside a value-plane word, of token slot u (0..31) of its
// 32-token block: u = 16c + 4g + j sits in bit 8j + 4c + g.  With this order a
// single AND with 0x01010101 << s extracts, as bytes, the four tokens that one
// int8 MFMA lane supplies (see the decode scan).
__host__ __device__ __forceinline__ int vbit(int u) { return 8 * (u & 3) + 4 * (u >> 4) + ((u >> 2) & 3); }
// Inverse: token slot held in bit position b.
__host__ __device__ __forceinline__ int vslot(int b) { return 16 * ((b >> 2) & 1) + 4 * (b & 3) + (b >> 3); }

// Min/max value codes of width 2 or 4 are stored packed rather than as bit
// planes: word h of a 32-token block holds the tokens (32/b) h + i, i < 32/b,
// with the code of token i in bits 8 (i % 4) + b (i / 4) .. + b - 1, so an AND
// leaves whole codes in byte lanes.  Width 1 is the same as one bit plane, and
// width 3 and the Lloyd-Max (MSE) value codes keep bit planes.
__host__ __device__ constexpr bool packed_value_codes(bool mse, int bits) { return !mse && (bits == 2 || bits == 4); }

// Code of token slot u (0..31) of a block from its `bits` value words.
template <int BITS, bool PACKED>
__device__ __forceinline__ uint32_t value_code(const uint32_t (&w)[BITS], int u) {
  if (PACKED) {
    constexpr int per = 32 / BITS;
    const int i = u % per;
    return (w[u / per] >> (8 * (i & 3) + BITS * (i >> 2))) & ((1u << BITS) - 1u);
  }
  uint32_t c = 0;
#pragma unroll
  for (int p = 0; p < BITS; ++p) c |= ((w[p] >> vbit(u)) & 1u) << p;
  return c;
}

// Bit-plane words (bit p of token u in bit vbit(u) of word p) -> packed words,
// for BITS = 2 or 4.  Byte j of every word is handled in place.
template <int BITS>
__device__ __forceinline__ void planes_to_packed(const uint32_t (&pl)[BITS], uint32_t (&out)[BITS]) {
  static_assert(BITS == 2 || BITS == 4, "packed widths are 2 and 4");
  if (BITS == 2) {
    // token 16h + 4k + j: plane bit 8j + 4h + k -> packed word h, bits 8j + 2k + q
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t o = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        uint32_t t = (pl[q] >> (4 * h)) & 0x0f0f0f0fu;  // bit k of byte j
        t = (t | (t << 2)) & 0x33333333u;
        t = (t | (t << 1)) & 0x55555555u;             // bit k -> bit 2k
        o |= t << q;
      }
      out[h] = o;
    }
  } else {
    // token 8h + 4k + j: plane bit 8j + 4(h/2) + 2(h%2) + k -> packed word h,
    // bits 8j + 4k + q
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t o = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t t = (pl[q] >> (4 * (h >> 1) + 2 * (h & 1))) & 0x03030303u;
        t = (t | (t << 3)) & 0x11111111u;  // bit k -> bit 4k
        o |= t << q;
      }
      out[h] = o;
    }
  }
}

// Valid-token mask in the bit-plane order -> the matching bit mask of each
// packed word (all b bits of every valid token).
template <int BITS>
__device__ __forceinline__ void mask_to_packed(uint32_t vmask, uint32_t (&out)[BITS]) {
  uint32_t pl[BITS];
#pragma unroll
  for (int p = 0; p < BITS; ++p) pl[p] = vmask;
  planes_to_packed<BITS>(pl, out);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// C += A * B on a 16x16x32 bf16 MFMA.  Lane l holds A[l%16][8*(l/16) + e] and
// B[8*(l/16) + e][l%16] for e = 0..7 (element e in half e%2 of dword e/2), and
// receives C[4*(l/16) + r][l%16] in accumulator r.
__device__ __forceinline__ floatx4 mfma_bf16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float load_scalar(const void* p, int64_t i, int f16) {
  if (f16) return __half2float(reinterpret_cast<const __half*>(p)[i]);
  return reinterpret_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_scalar(void* p, int64_t i, float x, int f16) {
  if (f16)
    reinterpret_cast<__half*>(p)[i] = __float2half_rn(x);
  else
    reinterpret_cast<float*>(p)[i] = x;
}

// Compute units of the current device (queried once per device).
inline int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Reductions over the wave, the result in every lane, in registers only (no
// LDS round trip): DPP steps within each 16-lane row, then the gfx950
// cross-row lane swaps combine the four rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm 1,0,3,2
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm 2,3,0,1
  x = fmaxf(x, dpp_f<0x124>(x));  // row_ror 4
  x = fmaxf(x, dpp_f<0x128>(x));  // row_ror 8
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
  auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(u[0]), __uint_as_float(u[1]));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x128>(x);
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(u[0]) + __uint_as_float(u[1]);
}

}  // namespace tq
