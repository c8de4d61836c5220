// Split-context merge on gfx950: top-k over the union of per-shard candidate lists, and the
// log-sum-exp combination of partial attentions over disjoint key sets.
//
// Pages: "vLLM 首日支持 Mistral Large 4" (best2ai.com), Long context › DCP: each context shard
// keeps its own top-2048 candidates, a stable top-k merge over (score, position) pairs
// selects the row's top-k (a radix select over packed candidates), and partial attention
// outputs are merged through their LSE.
//
// Merge: one 1024-thread work-group per row.  Every valid candidate becomes one 64-bit key,
// (order-preserving image of the fp32 score) << 32 | (2^32 - 1 - position), so larger keys
// rank first and equal scores rank the lower position first; keys are distinct, so an LDS
// radix select (11-bit digits below the candidates' common leading bits) finds the k-th key
// exactly.  The chosen positions are then sorted ascending by a bitonic network in LDS.
#include "ml4_device.h"

namespace ml4 {

namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMergeMax = 16384;          // candidates per row held in LDS
constexpr int kMergeOutMax = 2048;        // top_k
constexpr int kDigitBits = 11;
constexpr uint32_t kFaultTopk = 1u << 1;
constexpr uint32_t kFaultNan = 1u << 2;

__device__ __forceinline__ uint32_t score_key(float f, bool& nan) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    nan = true;
    return 0u;
  }
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kMergeThreads) void k_topk_merge(MergeLaunch a) {
  __shared__ uint64_t keys[kMergeMax];
  __shared__ uint32_t hist[1 << kDigitBits];
  __shared__ int sel[kMergeOutMax];
  __shared__ int sh_n, sh_digit, sh_above;
  __shared__ unsigned long long sh_and, sh_or;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int K = a.top_k;
  int32_t* out = a.idx + (size_t)r * K;
  if (tid == 0) { sh_n = 0; sh_and = ~0ull; sh_or = 0ull; }
  __syncthreads();

  // 1. gather the valid candidates of every shard as packed keys
  bool nan = false, bad = false;
  uint64_t av = ~0ull, ov = 0ull;
  for (int s = 0; s < a.n_shards; ++s) {
    int len = a.cand_len[(size_t)r * a.n_shards + s];
    if (len < 0 || len > a.ld) { bad = true; len = max(0, min(len, (int)a.ld)); }
    const size_t base = ((size_t)r * a.n_shards + s) * a.ld;
    for (int i = tid; i < len; i += kMergeThreads) {
      const int pos = a.cand_pos[base + i];
      if (pos < 0) { bad = true; continue; }
      const uint64_t key = ((uint64_t)score_key(a.cand_scores[base + i], nan) << 32) |
                           (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
      const int slot = atomicAdd(&sh_n, 1);
      if (slot < kMergeMax) keys[slot] = key;
      av &= key;
      ov |= key;
    }
  }
  if (nan) raise_fault(a.fault, kFaultNan);
  if (bad) raise_fault(a.fault, kFaultTopk);
  atomicAnd(&sh_and, (unsigned long long)av);
  atomicOr(&sh_or, (unsigned long long)ov);
  __syncthreads();
  const int m = min(sh_n, kMergeMax);
  const int n_out = min(K, m);

  // 2. the n_out-th largest key (all keys are taken when m <= K)
  uint64_t kth = 0;
  if (m > K) {
    const uint64_t diff = sh_and ^ sh_or;
    int shift = diff ? 64 - __builtin_clzll(diff) : 0;
    uint64_t P = shift >= 64 ? 0 : (sh_and >> shift);
    int need = n_out;
    while (shift > 0) {
      const int w = min(kDigitBits, shift);
      const int nsh = shift - w;
      const int nb = 1 << w;
      for (int i = tid; i < nb; i += kMergeThreads) hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < m; i += kMergeThreads) {
        const uint64_t k = keys[i];
        if ((shift >= 64 ? 0 : (k >> shift)) == P)
          atomicAdd(&hist[(uint32_t)(k >> nsh) & (nb - 1)], 1u);
      }
      __syncthreads();
      // digit d with above(d) < need <= above(d) + hist[d], scanning from the top digit
      if (tid == 0) {
        int above = 0;
        for (int d = nb - 1; d >= 0; --d) {
          const int c = (int)hist[d];
          if (above + c >= need) { sh_digit = d; sh_above = above; break; }
          above += c;
        }
      }
      __syncthreads();
      P = (P << w) | (uint64_t)sh_digit;
      need -= sh_above;
      shift = nsh;
      __syncthreads();
    }
    kth = P;
  }

  // 3. positions of the chosen keys, then ascending order
  if (tid == 0) sh_n = 0;
  __syncthreads();
  for (int i = tid; i < m; i += kMergeThreads) {
    const uint64_t k = keys[i];
    if (m <= K || k >= kth) {
      const int slot = atomicAdd(&sh_n, 1);
      if (slot < kMergeOutMax) sel[slot] = (int)(0xFFFFFFFFu - (uint32_t)k);
    }
  }
  __syncthreads();
  int N = 1;
  while (N < n_out) N <<= 1;
  for (int i = n_out + tid; i < N; i += kMergeThreads) sel[i] = 0x7FFFFFFF;
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < N / 2; t += kMergeThreads) {
        const int i = 2 * stride * (t / stride) + (t % stride);
        const int j = i + stride;
        const int x = sel[i], y = sel[j];
        const bool up = (i & size) == 0;
        if ((x > y) == up) { sel[i] = y; sel[j] = x; }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < K; i += kMergeThreads) out[i] = i < n_out ? sel[i] : -1;
  if (tid == 0) a.len[r] = n_out;
}

// o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M), lse = M + ln sum (natural log).
__global__ __launch_bounds__(128) void k_lse_combine(LseCombineLaunch a) {
  const int r = blockIdx.x, h = blockIdx.y;
  const int H = a.n_heads, S = a.n_shards, D = a.head_dim;
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.lse_parts[((size_t)r * S + s) * H + h]);
  float L = 0.f;
  for (int s = 0; s < S; ++s) {
    const float l = a.lse_parts[((size_t)r * S + s) * H + h];
    L += (l == -__builtin_inff()) ? 0.f : expf(l - M);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  for (int d = threadIdx.x; d < D; d += 128) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float l = a.lse_parts[((size_t)r * S + s) * H + h];
      if (l == -__builtin_inff()) continue;
      acc += expf(l - M) * a.o_parts[(((size_t)r * S + s) * H + h) * D + d];
    }
    const float v = acc * inv;
    if (a.out_bf16)
      static_cast<__bf16*>(a.out)[((size_t)r * H + h) * D + d] = (__bf16)v;
    else
      static_cast<float*>(a.out)[((size_t)r * H + h) * D + d] = v;
  }
  if (a.lse && threadIdx.x == 0)
    a.lse[(size_t)r * H + h] = L > 0.f ? M + logf(L) : -__builtin_inff();
}

}  // namespace

hipError_t launch_topk_merge(const MergeLaunch& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  k_topk_merge<<<a.rows, kMergeThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_lse_combine(const LseCombineLaunch& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  k_lse_combine<<<dim3(a.rows, a.n_heads), 128, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace ml4
