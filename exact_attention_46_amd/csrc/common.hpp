// Device helpers shared by the attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element type codes, as in the C ABI.
constexpr int kBF16 = 0;
constexpr int kFP16 = 1;

// D = A * B + C on one 32x32x16 MFMA tile with fp32 accumulation. A and B each
// carry 8 packed 16-bit elements per lane (bf16 when DT == kBF16, else fp16).
// Lane l supplies row (l % 32) of A / column (l % 32) of B and the k-slots
// 8 * (l / 32) .. +7; the accumulator element e of lane l is row
// 8 * (e / 4) + 4 * (l / 32) + (e % 4), column l % 32.
template <int DT>
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Two fp32 values -> one dword holding two 16-bit values (x in the low half),
// rounded to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  if constexpr (DT == kBF16) {
    bf16x2_t h = __builtin_convertvector((f32x2_t){x, y}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
  } else {
    f16x2_t h = __builtin_convertvector((f32x2_t){x, y}, f16x2_t);
    return __builtin_bit_cast(uint32_t, h);
  }
}

// The value of the partner lane (l ^ 32) combined with this lane's value.
__device__ __forceinline__ float max_with_partner32(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  return x + __shfl_xor(x, 32, 64);
}

// Lane-halves of two dwords: {lo16(a), lo16(b)} and {hi16(a), hi16(b)}.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// acc + lo + hi of a dword holding two 16-bit values (exact products with 1.0).
template <int DT>
__device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, packed),
                                  __builtin_bit_cast(f16x2_t, 0x3c003c00u), acc, false);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace mi355attn
