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

// This lane's value combined with that of its partner lane l ^ 32, through
// v_permlane32_swap (a VALU lane swap between the two 32-lane halves, no LDS
// round trip). Passing x as both operands, result[0] holds, in lanes 32..63,
// the low half's values and result[1] holds, in lanes 0..31, the high half's
// values; in the other lanes each holds x itself, so combining the two gives
// f(x_l, x_{l^32}) in every lane.
__device__ __forceinline__ float max_with_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Buffer resource for a raw (stride 0) buffer of `bytes` bytes at `base`. Loads
// through it at byte offsets >= bytes return zero instead of touching memory,
// which is how ragged tiles are zero-filled without per-row branches.
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer format word

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

// 16-byte load at byte offset `off` (zero when off lies past the buffer end).
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Cache-policy bits of a buffer load: 0 is the default; kNonTemporal marks a
// stream read once (the data need not stay in the caches).
constexpr int kCacheDefault = 0;
constexpr int kNonTemporal = 2;

// 16-byte load from a raw buffer straight into LDS: lane p's 16 bytes land at
// lds_base + 16 * p (lds_base must be the same for the whole wave); offsets
// past the buffer end write zeros. Completion is counted by vmcnt.
template <int Policy = kCacheDefault>
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                               uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0, Policy);
}

typedef __attribute__((ext_vector_type(4))) short s16x4_t;

// Transposing LDS read of four 16-bit values (gfx950 ds_read_b64_tr_b16).
// Within each 16-lane group, source lane j = 4k + a supplies the address of 4
// consecutive elements; output lane i = 4a + c receives element c of source
// lanes 4k + a for k = 0..3 (element k of the result).
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// The same transposing read for kernels that stage tiles with buffer loads to
// LDS. The compiler's wait insertion treats an LDS read that carries no alias
// scope as possibly reading bytes a buffer load to LDS still in flight writes,
// and precedes it with a wait for all outstanding vector-memory loads. The
// restrict-qualified parameter gives the read a scope of its own, which lifts
// that wait; the caller guarantees (with its own waits and barriers) that the
// bytes it reads have landed.
__device__ __forceinline__ u32x2_t lds_read_tr16_staged(const lds_s16x4_t* __restrict__ p) {
  return __builtin_bit_cast(u32x2_t,
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4_t*>(p)));
}

// 32-bit LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Four groups of four transposing LDS reads (ds_read_b64_tr_b16, lane layout
// as in lds_read_tr16): out[4 * j + i] is read at LDS address base[j] + i * STEP.
// The group ends by waiting for all of this wave's LDS accesses, so the results
// are valid when it returns. It is written in assembly because the compiler
// cannot tell these reads apart from the buffer loads to LDS still in flight
// (which target other LDS bytes) and would otherwise make them wait for every
// outstanding vector-memory load first.
template <int STEP>
__device__ __forceinline__ void lds_read_tr16_x16(u32x2_t (&out)[16], const uint32_t (&base)[4]) {
  static_assert(3 * STEP < 65536, "ds offset field is 16 bits");
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:%20\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:%21\n\t"
      "ds_read_b64_tr_b16 %3, %16 offset:%22\n\t"
      "ds_read_b64_tr_b16 %4, %17\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:%20\n\t"
      "ds_read_b64_tr_b16 %6, %17 offset:%21\n\t"
      "ds_read_b64_tr_b16 %7, %17 offset:%22\n\t"
      "ds_read_b64_tr_b16 %8, %18\n\t"
      "ds_read_b64_tr_b16 %9, %18 offset:%20\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:%21\n\t"
      "ds_read_b64_tr_b16 %11, %18 offset:%22\n\t"
      "ds_read_b64_tr_b16 %12, %19\n\t"
      "ds_read_b64_tr_b16 %13, %19 offset:%20\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:%21\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:%22\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]),
        "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7]), "=&v"(out[8]), "=&v"(out[9]),
        "=&v"(out[10]), "=&v"(out[11]), "=&v"(out[12]), "=&v"(out[13]), "=&v"(out[14]),
        "=&v"(out[15])
      : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "i"(STEP), "i"(2 * STEP),
        "i"(3 * STEP)
      : "memory");
}

// Two groups of four transposing LDS reads, as lds_read_tr16_x16.
template <int STEP>
__device__ __forceinline__ void lds_read_tr16_x8(u32x2_t (&out)[8], const uint32_t (&base)[2]) {
  static_assert(3 * STEP < 65536, "ds offset field is 16 bits");
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %9\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:%10\n\t"
      "ds_read_b64_tr_b16 %6, %9 offset:%11\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]),
        "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7])
      : "v"(base[0]), "v"(base[1]), "i"(STEP), "i"(2 * STEP), "i"(3 * STEP)
      : "memory");
}

// Waits for every outstanding memory operation of this wave (vector memory,
// LDS, scalar memory). Placed where those operations must be complete anyway
// (before a barrier that publishes LDS stores fed by global loads), it also
// tells the compiler's wait-count tracking that nothing is pending afterwards.
// The waits below are also scheduling barriers: LDS data written by buffer
// loads to LDS is only visible after the wait, which the compiler cannot see.
__device__ __forceinline__ void wait_all_memory() {
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; a field at its maximum does not wait).
// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
  __builtin_amdgcn_sched_barrier(0);
}
// Wait until at most N vector memory operations and no LDS operation of this
// wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkmcnt0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
  __builtin_amdgcn_sched_barrier(0);
}
// Wait until every LDS operation of this wave has completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace mi355attn
