// KV-cache writes on gfx950: quantise and pack new tokens into the 132-byte indexer rows and
// the latent rows read by the rest of the path (656-byte fp8_ds_mla, and the two second
// layouts: 1,152-byte bf16 and 576-byte plain E4M3 with one per-tensor scale).
//
// Pages: "vLLM 首日支持 Mistral Large 4" (best2ai.com), ROCm implementation details ›
// AITER 上的 DSA 索引器 (an FP8 indexer key with a single scale per key, 132 bytes per token)
// and › FP8 潜在缓存 (fp8_ds_mla: 512 FP8 values with four scales, one per 128, and 64 bf16
// RoPE values, 656 bytes per token).  The quantiser is the plain symmetric one: per scale
// group scale = amax / 448 and code = E4M3(x / scale), round to nearest even, clamped to
// +-448 (binary32 arithmetic); an all-zero group stores scale 0 and zero codes.
//
// Index rows: 16 lanes per token (four tokens per wave), each converting eight of the 128
// values; the scale is the maximum over the token's 16 lanes.  Latent rows: one wave per
// token, each lane converting eight of the 512 values; the 16 lanes of a 128-value group
// reduce their maximum with xor shuffles, and lanes 0..15 copy the RoPE bytes.  Each lane
// reads its eight source values with one 16-byte load (bf16) or two (fp32).  Both are
// streams: 256 B (bf16 key) or 1,160 B (bf16 latent + RoPE) read and 132 or 656 B written
// per token.
//
// Second layouts [same page, › FP8 潜在缓存: the uncompressed bf16 row and the per-tensor-scale
// E4M3 row]: the bf16 row takes the latents rounded to nearest even and the RoPE bits as
// given; the E4M3 row takes code = E4M3(x / kv_scale), clamped to +-448 and rounded to
// nearest even in binary32, for the latents and the RoPE values alike.  Same one wave per
// token, eight latents per lane, lanes 0..15 on the RoPE values.
#include "ml4_device.h"

namespace ml4 {

namespace {

constexpr int kIdxRowBytes = 132;
constexpr int kLatRowBytes = 656;
constexpr int kBf16RowBytes = 1152;
constexpr int kE4m3RowBytes = 576;
constexpr int kWavesPerWg = 4;
constexpr float kE4m3Max = 448.0f;
constexpr uint32_t kFaultSlot = 1u << 0;
constexpr uint32_t kFaultRange = 1u << 4;

// Eight consecutive source values (element i, a multiple of 8) as binary32, with one 16-byte
// load for bf16 sources and two for fp32.
template <typename T>
__device__ __forceinline__ void load8(const void* p, size_t i, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p) + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
  }
}

// Two binary32 values inside [-448, 448] -> two OCP E4M3 codes (round to nearest even) in
// the low 16 bits.
__device__ __forceinline__ uint32_t to_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// binary32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float quantise_input(float x, float scale) {
  if (scale == 0.f) return 0.f;
  return fminf(fmaxf(x / scale, -kE4m3Max), kE4m3Max);
}

// Resolves the destination row of `token`; -1 = skip (negative slot: padding token).
__device__ __forceinline__ int64_t dest_slot(const CacheWriteLaunch& a, int64_t token) {
  const int64_t slot = a.slot_mapping[token];
  if (slot < 0) return -1;
  if (slot >= a.capacity) {
    raise_fault(a.fault, kFaultSlot);
    return -1;
  }
  return slot;
}

// Index rows: 16 lanes per token (four tokens per wave), eight values per lane.
constexpr int kIdxTokPerWg = kWavesPerWg * kWave / 16;
template <typename T>
__global__ __launch_bounds__(kWavesPerWg * kWave) void k_index_write(CacheWriteLaunch a) {
  const int l16 = threadIdx.x & 15;
  const int64_t token = (int64_t)blockIdx.x * kIdxTokPerWg + (threadIdx.x >> 4);
  if (token >= a.n_tokens) return;        // whole 16-lane groups leave together
  const int64_t slot = dest_slot(a, token);
  if (slot < 0) return;
  float x[8];
  load8<T>(a.src, (size_t)token * 128 + 8 * l16, x);
  bool finite = true;
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    finite &= __builtin_isfinite(x[e]);
    m = fmaxf(m, fabsf(x[e]));
  }
  if (__any(!finite) && (threadIdx.x & (kWave - 1)) == 0) raise_fault(a.fault, kFaultRange);
  // maximum over the token's 16 lanes
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float scale = m / kE4m3Max;
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = to_e4m3x2(quantise_input(x[4 * h], scale), quantise_input(x[4 * h + 1], scale));
    const uint32_t hi = to_e4m3x2(quantise_input(x[4 * h + 2], scale), quantise_input(x[4 * h + 3], scale));
    w[h] = lo | (hi << 16);
  }
  uint8_t* row = static_cast<uint8_t*>(a.pool) + slot * kIdxRowBytes;
  *reinterpret_cast<u32x2*>(row + 8 * l16) = u32x2{w[0], w[1]};
  if (l16 == 0) *reinterpret_cast<float*>(row + 128) = scale;
}

template <typename T>
__global__ __launch_bounds__(kWavesPerWg * kWave) void k_latent_write(CacheWriteLaunch a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t token = (int64_t)blockIdx.x * kWavesPerWg + (threadIdx.x >> 6);
  if (token >= a.n_tokens) return;
  const int64_t slot = dest_slot(a, token);
  if (slot < 0) return;
  float x[8];
  load8<T>(a.src, (size_t)token * 512 + 8 * lane, x);
  bool finite = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) finite &= __builtin_isfinite(x[e]);
  if (__any(!finite) && lane == 0) raise_fault(a.fault, kFaultRange);
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  // maximum over the 16 lanes of this lane's 128-value group
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float scale = m / kE4m3Max;
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = to_e4m3x2(quantise_input(x[4 * h], scale), quantise_input(x[4 * h + 1], scale));
    const uint32_t hi = to_e4m3x2(quantise_input(x[4 * h + 2], scale), quantise_input(x[4 * h + 3], scale));
    w[h] = lo | (hi << 16);
  }
  uint8_t* row = static_cast<uint8_t*>(a.pool) + slot * kLatRowBytes;
  *reinterpret_cast<u32x2*>(row + 8 * lane) = u32x2{w[0], w[1]};
  if ((lane & 15) == 0) *reinterpret_cast<float*>(row + 512 + 4 * (lane >> 4)) = scale;
  if (a.rope_dim && lane < 16) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a.rope) +
                                                     (size_t)token * 128 + 8 * lane);
    *reinterpret_cast<uint2*>(row + 528 + 8 * lane) = v;
  }
}

template <typename T>
__global__ __launch_bounds__(kWavesPerWg * kWave) void k_latent_write_bf16(CacheWriteLaunch a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t token = (int64_t)blockIdx.x * kWavesPerWg + (threadIdx.x >> 6);
  if (token >= a.n_tokens) return;
  const int64_t slot = dest_slot(a, token);
  if (slot < 0) return;
  float x[8];
  load8<T>(a.src, (size_t)token * 512 + 8 * lane, x);
  uint32_t w[4];
  bool finite = true;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    finite &= __builtin_isfinite(x[2 * e]) && __builtin_isfinite(x[2 * e + 1]);
    w[e] = bf16_bits(x[2 * e]) | (bf16_bits(x[2 * e + 1]) << 16);
  }
  if (__any(!finite) && lane == 0) raise_fault(a.fault, kFaultRange);
  uint8_t* row = static_cast<uint8_t*>(a.pool) + slot * kBf16RowBytes;
  *reinterpret_cast<u32x4*>(row + 16 * lane) = u32x4{w[0], w[1], w[2], w[3]};
  if (a.rope_dim && lane < 16) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a.rope) +
                                                     (size_t)token * 128 + 8 * lane);
    *reinterpret_cast<uint2*>(row + 1024 + 8 * lane) = v;
  }
}

template <typename T>
__global__ __launch_bounds__(kWavesPerWg * kWave) void k_latent_write_e4m3(CacheWriteLaunch a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t token = (int64_t)blockIdx.x * kWavesPerWg + (threadIdx.x >> 6);
  if (token >= a.n_tokens) return;
  const int64_t slot = dest_slot(a, token);
  if (slot < 0) return;
  const float scale = a.kv_scale;
  float x[8];
  load8<T>(a.src, (size_t)token * 512 + 8 * lane, x);
  bool finite = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) finite &= __builtin_isfinite(x[e]);
  float r[4] = {0.f, 0.f, 0.f, 0.f};
  const bool has_rope = a.rope_dim && lane < 16;
  if (has_rope) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(static_cast<const __bf16*>(a.rope) +
                                                      (size_t)token * 64 + 4 * lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (float)v[e];
      finite &= __builtin_isfinite(r[e]);
    }
  }
  if (__any(!finite) && lane == 0) raise_fault(a.fault, kFaultRange);
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = to_e4m3x2(quantise_input(x[4 * h], scale), quantise_input(x[4 * h + 1], scale));
    const uint32_t hi = to_e4m3x2(quantise_input(x[4 * h + 2], scale), quantise_input(x[4 * h + 3], scale));
    w[h] = lo | (hi << 16);
  }
  uint8_t* row = static_cast<uint8_t*>(a.pool) + slot * kE4m3RowBytes;
  *reinterpret_cast<u32x2*>(row + 8 * lane) = u32x2{w[0], w[1]};
  if (has_rope) {
    const uint32_t lo = to_e4m3x2(quantise_input(r[0], scale), quantise_input(r[1], scale));
    const uint32_t hi = to_e4m3x2(quantise_input(r[2], scale), quantise_input(r[3], scale));
    *reinterpret_cast<uint32_t*>(row + 512 + 4 * lane) = lo | (hi << 16);
  }
}

template <typename T>
hipError_t launch_typed(const CacheWriteLaunch& a, hipStream_t st) {
  constexpr int NT = kWavesPerWg * kWave;
  const dim3 grid((unsigned)((a.n_tokens + kWavesPerWg - 1) / kWavesPerWg));
  if (a.latent && a.bf16_rows)
    k_latent_write_bf16<T><<<grid, NT, 0, st>>>(a);
  else if (a.latent && a.e4m3_rows)
    k_latent_write_e4m3<T><<<grid, NT, 0, st>>>(a);
  else if (a.latent)
    k_latent_write<T><<<grid, NT, 0, st>>>(a);
  else
    k_index_write<T><<<dim3((unsigned)((a.n_tokens + kIdxTokPerWg - 1) / kIdxTokPerWg)), NT, 0,
                        st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteLaunch& a, hipStream_t st) {
  if (a.n_tokens == 0) return hipSuccess;
  return a.bf16 ? launch_typed<__bf16>(a, st) : launch_typed<float>(a, st);
}

}  // namespace ml4
