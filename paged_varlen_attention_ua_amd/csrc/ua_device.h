// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ua_internal.h"

namespace ua {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16x16x32 MFMA on 16-bit inputs held as 4 dwords per lane.
template <int QT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (QT == UA_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// 32x32x16 MFMA on 16-bit inputs held as 4 dwords per lane.
template <int QT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (QT == UA_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// Two fp32 -> packed pair of QT (round to nearest even).
template <int QT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (QT == UA_F16) {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// acc + lo + hi of a packed pair of QT values (one v_dot2c against (1, 1)):
// the sum of p values exactly as rounded for the PV MFMA.
template <int QT>
__device__ __forceinline__ float add_pair(uint32_t pk, float acc) {
  if constexpr (QT == UA_F16) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk),
                                  __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
  }
}

// Byte permute: result byte i = byte sel_i of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two E4M3 codes (bytes 0,1 when hi == false, bytes 2,3 otherwise) -> packed QT pair.
// OCP e4m3fn (FNUZ == false): every value is exactly representable in fp16 and
// bf16, so this is exact.
// e4m3fnuz (FNUZ == true): the code of a value is the e4m3fn code of twice that
// value, except for 0x7F / 0xFF (+-240, NaN in e4m3fn) and 0x80 (NaN; -0 in
// e4m3fn, never produced by a quantiser).  The result is TWICE the fnuz value
// (the caller folds the factor 1/2 into its fp32 scales): the magnitudes are
// converted as e4m3fn, the NaN of 0x7F is clamped to 480 by an unsigned 16-bit
// minimum (every finite e4m3fn magnitude is <= 448 < 480, and a non-negative
// float orders like its bits), and the sign bits are put back.  Exact as well.
template <int QT, bool FNUZ = false>
__device__ __forceinline__ uint32_t fp8x2_to(uint32_t v, bool hi) {
  if constexpr (FNUZ) {
    const uint32_t mag = fp8x2_to<QT, false>(v & 0x7F7F7F7Fu, hi);
    const u16x2 cap = QT == UA_F16 ? u16x2{0x5F80, 0x5F80} : u16x2{0x43F0, 0x43F0};
    const u16x2 m = __builtin_elementwise_min(__builtin_bit_cast(u16x2, mag), cap);
    // sign of byte 0/2 -> bit 15, of byte 1/3 -> bit 31
    const uint32_t sgn = perm_b32(0u, v, hi ? 0x030c020cu : 0x010c000cu) & 0x80008000u;
    return __builtin_bit_cast(uint32_t, m) | sgn;
  } else if constexpr (QT == UA_F16) {
    return __builtin_bit_cast(uint32_t,
                              hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, true)
                                 : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false));
  } else {
    return __builtin_bit_cast(uint32_t,
                              hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true)
                                 : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false));
  }
}

// 8 E4M3 codes (2 dwords) -> 8 QT values (4 dwords), order preserved.
template <int QT, bool FNUZ = false>
__device__ __forceinline__ u32x4 fp8x8_to(u32x2 v) {
  u32x4 r;
  r[0] = fp8x2_to<QT, FNUZ>(v[0], false);
  r[1] = fp8x2_to<QT, FNUZ>(v[0], true);
  r[2] = fp8x2_to<QT, FNUZ>(v[1], false);
  r[3] = fp8x2_to<QT, FNUZ>(v[1], true);
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh from one base-2 exponential: tanh|x| = (1 - e) / (1 + e), e = 2^(-2|x| log2 e).
__device__ __forceinline__ float tanh_fast(float x) {
  float e = fast_exp2(-2.0f * kLog2e * __builtin_fabsf(x));
  float t = (1.0f - e) * fast_rcp(1.0f + e);
  return __builtin_copysignf(t, x);
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  uint32_t t = __umulhi(n, f.m);
  return (uint32_t)(((uint64_t)t + n) >> f.l);
}

// Sequence owning query-block slot qb: the last s with cu[s] / bq + s <= qb
// (slots of sequence s start at cu[s] / bq + s; a sequence with no query
// token owns exactly one slot, which finds no token and exits).
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int num_seqs, int qb,
                                        int bq) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] / bq + mid <= qb)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_sum_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

}  // namespace ua
