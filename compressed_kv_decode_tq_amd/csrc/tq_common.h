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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace tq
