// Device-side helpers shared by the gfx950 kernels: vector types, MFMA wrappers, exact fp8
// decoding, wave reductions and fault reporting.  gfx950 only (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ml4_launch.h"

namespace ml4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 16-byte vector that may sit at any 4-byte boundary (132-byte indexer rows).
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(16x16 f32) += A(16x128 e4m3) * B(128x16 e4m3).  Lane l holds A row l%16 and B column
// l%16, bytes 32*(l/16) .. +31 of the K axis (the same K order on both sides); D lane l
// holds rows 4*(l/16)+j, column l%16.  Products of e4m3 values are exact in fp32.
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16); lane l: A row / B column l%16, K elements
// 8*(l/16) .. +7; D lane l: rows 4*(l/16)+j, column l%16.
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16 f32) += A(16x32 f16) * B(32x16 f16); same lane layout as mfma_bf16.
__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const f16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Four OCP e4m3 codes (one dword) -> four fp16, exactly (e4m3 values are fp16 values).
__device__ __forceinline__ f16x4 e4m3x4_to_f16(uint32_t w) {
  f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  f16x4 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
  return r;
}

// Four OCP e4m3 codes (one dword) -> four bf16, exactly (every e4m3 value is a bf16 value).
__device__ __forceinline__ bf16x4 e4m3x4_to_bf16(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  bf16x4 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
  return r;
}

// ReLU as one integer max on the IEEE bits: negative floats (sign bit set) compare below
// 0, -0 maps to +0, non-negative values are unchanged.  (A float max would first quiet
// signalling NaNs with an extra instruction per element.)
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ void raise_fault(uint32_t* fault, uint32_t bit) {
  if (fault) atomicOr(fault, bit);
}

// SSMax multiplier s * ln(p + 1) (1 when s <= 0).
__device__ __forceinline__ float ssmax_mult(float s, int pos) {
  return s > 0.f ? s * logf((float)pos + 1.0f) : 1.0f;
}

// Request owning query row r: the b with q_start[b] <= r < q_start[b+1].
__device__ __forceinline__ int request_of(const int32_t* q_start, int batch, int r) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same, found by a whole wave in one round of loads (every lane passes the same r):
// q_start is non-decreasing, so the owner is the number of b in [1, batch) with
// q_start[b] <= r.
__device__ __forceinline__ int request_of_wave(const int32_t* q_start, int batch, int r) {
  const int lane = threadIdx.x & (kWave - 1);
  int n = 0;
  for (int base = 1; base < batch; base += kWave) {
    const int i = base + lane;
    n += __popcll(__ballot(i < batch && q_start[i] <= r));
  }
  return n;
}

}  // namespace ml4
