// Measurement probes: the rates this GPU reaches on a plain streaming read and on
// back-to-back independent MFMAs, the "achievable" peaks the step's kernels are compared
// against beside the datasheet ones.  Not part of the attention path.
#include "ml4_device.h"

namespace ml4 {
namespace {

// Every lane reads 16-byte vectors with a grid-stride loop; one partial sum per work-group
// keeps the loads live.
__global__ __launch_bounds__(256) void k_probe_read(const u32x4* buf, size_t n16, float* sink) {
  u32x4 acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * 256 * 4;
  for (size_t i = (size_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + 256 * u < n16 ? buf[i + 256 * u] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[blockIdx.x] = 1.0f;
}

// 16 independent accumulation chains of v_mfma_f32_16x16x32_f16 (KIND 0) or
// v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 (KIND 1) per wave.
template <int KIND>
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float* sink) {
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int l = threadIdx.x;
  if constexpr (KIND == 0) {
    f16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a[e] = (_Float16)(0.001f * (l + e)); b[e] = (_Float16)(0.5f * e); }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = mfma_f16(a, b, acc[j]);
  } else {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a[e] = 0x38383838 + l; b[e] = 0x30303030 + e; }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = mfma_fp8(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += acc[j][0] + acc[j][3];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

}  // namespace
}  // namespace ml4

extern "C" int ml4_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
  if (!buf || !sink || (bytes & 15) || ((uintptr_t)buf & 15)) return -1;
  ml4::k_probe_read<<<2048, 256, 0, stream>>>(static_cast<const ml4::u32x4*>(buf), bytes / 16,
                                              sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int ml4_probe_mfma(int32_t kind, int32_t iters, float* sink, hipStream_t stream) {
  if (!sink || iters < 1 || (kind != 0 && kind != 1)) return -1;
  // 8 waves per SIMD on 256 CUs, 4 rounds of work-groups
  if (kind == 0) ml4::k_probe_mfma<0><<<256 * 8 * 4, 256, 0, stream>>>(iters, sink);
  else ml4::k_probe_mfma<1><<<256 * 8 * 4, 256, 0, stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
