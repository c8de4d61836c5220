// Exact top-k per query row on gfx950.
//
// Pages: "vLLM 首日支持 Mistral Large 4" (best2ai.com), ROCm implementation details › 专用解码
// (the persistent decode kernel computes an exact top-2048) and Long context › DCP (a stable
// top-k merge; radix select over packed (score, id) candidates; top-k compaction: padded -1
// slots bounded by topk_length).
//
// Selection is integer work on the order-preserving u32 image of each fp32 score (-0 folded
// onto +0, NaN mapped below -inf), so it is exact and deterministic:
//   1. AND/OR reduction of the keys: the leading bits common to every candidate are skipped.
//   2. Radix passes of up to 11 bits below that prefix: an LDS histogram, a block-wide
//      suffix scan to find the digit holding the k-th key, until the k-th key's bits are all
//      known (or its bucket is taken whole).
//   3. Ordered compaction in ascending t: keys above the threshold are kept; keys equal to it
//      are kept lowest-t first until k are chosen (wave ballots + block prefix sums).
// Rows up to 131,072 positions first narrow the row to an LDS candidate list with a
// threshold taken from a sample (one read of the row), and run steps 2-3 on that list; the
// streaming form above is their fallback when the list misses.  Rows up to 32,768 positions
// hold the whole row in registers (32 keys per thread), so the sample and the candidate
// pass read no memory.  Longer rows take two launches: many work-groups per row
// filter their chunks against the sampled threshold into per-chunk lists, then one
// work-group per row selects from the concatenated lists.
#include "ml4_device.h"

namespace ml4 {

namespace {

constexpr int kRowThreads = 1024;
constexpr int kCacheKeys = 32768;
constexpr int kBigChunk = 4096;
constexpr int kBigThreads = 256;
constexpr int kMaxDigitBits = 11;
constexpr uint32_t kFaultNan = 1u << 2;
constexpr uint32_t kFaultQpos = 1u << 3;

__device__ __forceinline__ uint32_t order_key(float f, bool& is_nan) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    is_nan = true;
    return 0u;
  }
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t digit_prefix(uint32_t key, int shift) {
  return (uint64_t)key >> shift;   // shift in [0, 32]
}

// Exclusive prefix sum over the block; *total receives the block sum.  Every thread of the
// block must call it.  sh needs NT/64 ints.
template <int NT>
__device__ int block_exclusive_scan(int v, int* total, int* sh) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int t = lane < NW ? sh[lane] : 0;
#pragma unroll
    for (int d = 1; d < NW; d <<= 1) {
      const int y = __shfl_up(t, d);
      if (lane >= d) t += y;
    }
    if (lane < NW) sh[lane] = t;
  }
  __syncthreads();
  const int off = wave ? sh[wave - 1] : 0;
  *total = sh[NW - 1];
  __syncthreads();
  return off + x - v;
}

// Given a histogram (nb bins, descending order of digit = descending key), find the digit d
// with above(d) < need <= above(d) + hist[d].  Writes {d, above(d), hist[d]} to out.  Thread
// i scans the digits nb-1-B i .. nb-B-B i (B = 2,048 / NT) in descending order.
template <int NT>
__device__ void find_digit(const uint32_t* hist, int nb, int need, int* out, int* sh) {
  constexpr int B = (1 << kMaxDigitBits) / NT;
  static_assert(B >= 1 && B * NT == (1 << kMaxDigitBits), "whole digits per thread");
  int c[B];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int d = nb - 1 - (B * (int)threadIdx.x + j);
    c[j] = d >= 0 ? (int)hist[d] : 0;
    sum += c[j];
  }
  int total;
  int ex = block_exclusive_scan<NT>(sum, &total, sh);
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int d = nb - 1 - (B * (int)threadIdx.x + j);
    if (d >= 0 && ex < need && need <= ex + c[j]) {
      out[0] = d; out[1] = ex; out[2] = c[j];
    }
    ex += c[j];
  }
  __syncthreads();
}

// Row r's case: 0 = a selection over n > k positions, 1 = a position outside its request,
// 2 = n <= k (the row is returned whole).  *n_out = p + 1 when the position is valid.
// Called by whole waves.
__device__ __forceinline__ int row_kind(const TopkLaunch& a, int r, int* n_out) {
  const SeqView& s = a.s;
  const int b = request_of_wave(s.q_start, s.batch, r);
  const int p = s.q_pos[r];
  if (p < 0 || p >= s.seq_lens[b] || p >= s.max_seq_len || (int64_t)p >= a.ld) return 1;
  *n_out = p + 1;
  return p + 1 <= a.top_k ? 2 : 0;
}

// row_kind, plus the output of a row that needs no selection; true for a selection row.
__device__ __forceinline__ bool row_prologue(const TopkLaunch& a, int r, int* n_out) {
  int n = 0;
  const int kind = row_kind(a, r, &n);
  int32_t* out = a.idx + (size_t)r * a.top_k;
  if (kind == 1) {
    for (int i = threadIdx.x; i < a.top_k; i += blockDim.x) out[i] = -1;
    if (threadIdx.x == 0) {
      a.len[r] = 0;
      raise_fault(a.fault, kFaultQpos);
    }
    return false;
  }
  if (kind == 2) {
    for (int i = threadIdx.x; i < a.top_k; i += blockDim.x) out[i] = i < n ? i : -1;
    if (threadIdx.x == 0) a.len[r] = n;
    return false;
  }
  *n_out = n;
  return true;
}

// ------------------------------------------------------------------ one work-group per row
// Scores are read as float4 (rows are 16-byte aligned and ld % 4 == 0, so the vector holding
// the last candidate lies inside the row), U vectors per thread in flight per batch.
constexpr int kU = 4;

template <bool CACHE>
__device__ __forceinline__ void load_keys(const float* row, const uint32_t* kc, int i4,
                                          uint32_t k[4]) {
  if (CACHE) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(kc + 4 * i4);
    k[0] = v[0]; k[1] = v[1]; k[2] = v[2]; k[3] = v[3];
  } else {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + 4 * i4);
    bool nn = false;
    k[0] = order_key(v[0], nn); k[1] = order_key(v[1], nn);
    k[2] = order_key(v[2], nn); k[3] = order_key(v[3], nn);
  }
}

// Calls f(t, key) for every candidate t < n, threads striding over float4 vectors.
template <bool CACHE, typename F>
__device__ __forceinline__ void for_each_key(const float* row, const uint32_t* kc, int n, F&& f) {
  const int n4 = (n + 3) >> 2;
  for (int base = threadIdx.x; base < n4; base += kRowThreads * kU) {
    uint32_t k[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kRowThreads;
      if (i4 < n4) load_keys<CACHE>(row, kc, i4, k[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kRowThreads;
      if (i4 >= n4) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * i4 + e < n) f(4 * i4 + e, k[u][e]);
    }
  }
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Exact selection for row r with n > K candidates, streaming the row (CACHE: keys kept in
// kcache after the first read).  Called by every thread of a kRowThreads work-group.
template <bool CACHE>
__device__ void row_select_exact(const TopkLaunch& a, int r, int n, uint32_t* kcache) {
  constexpr int NW = kRowThreads / kWave;
  __shared__ uint32_t hist[1 << kMaxDigitBits];
  __shared__ int sh_scan[NW];
  __shared__ uint32_t sh_and[NW], sh_or[NW];
  __shared__ int sh_sel[4];
  __shared__ int sh_nan;
  __shared__ int sh_gt[NW], sh_eq[NW];

  const int K = a.top_k;
  const float* row = a.scores + (size_t)r * a.ld;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int n4 = (n + 3) >> 2;

  // 1. common leading bits of every candidate key (and the LDS key cache)
  uint32_t av = ~0u, ov = 0u;
  bool any_nan = false;
  for (int base = tid; base < n4; base += kRowThreads * kU) {
    f32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kRowThreads;
      if (i4 < n4) v[u] = *reinterpret_cast<const f32x4*>(row + 4 * i4);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kRowThreads;
      if (i4 >= n4) continue;
      uint32_t k[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool nn = false;
        k[e] = order_key(v[u][e], nn);
        if (4 * i4 + e < n) {
          any_nan |= nn;
          av &= k[e];
          ov |= k[e];
        }
      }
      if (CACHE) *reinterpret_cast<u32x4*>(kcache + 4 * i4) = u32x4{k[0], k[1], k[2], k[3]};
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    av &= (uint32_t)__shfl_xor((int)av, m);
    ov |= (uint32_t)__shfl_xor((int)ov, m);
  }
  if (tid == 0) sh_nan = 0;
  if (lane == 0) { sh_and[wave] = av; sh_or[wave] = ov; }
  __syncthreads();
  if (any_nan) sh_nan = 1;
  av = ~0u; ov = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) { av &= sh_and[w]; ov |= sh_or[w]; }
  __syncthreads();
  if (tid == 0 && sh_nan) raise_fault(a.fault, kFaultNan);

  const uint32_t diff = av ^ ov;
  int shift = diff ? 32 - __builtin_clz(diff) : 0;   // bits >= shift are common
  uint64_t P = digit_prefix(av, shift);
  int need = K;

  // 2. radix passes below the common prefix
  while (shift > 0) {
    const int w = min(kMaxDigitBits, shift);
    const int nsh = shift - w;
    const int nb = 1 << w;
    for (int i = tid; i < nb; i += kRowThreads) hist[i] = 0u;
    __syncthreads();
    for_each_key<CACHE>(row, kcache, n, [&](int, uint32_t k) {
      if (digit_prefix(k, shift) == P) atomicAdd(&hist[(k >> nsh) & (nb - 1)], 1u);
    });
    __syncthreads();
    find_digit<kRowThreads>(hist, nb, need, sh_sel, sh_scan);
    const int d = sh_sel[0], above = sh_sel[1], cnt = sh_sel[2];
    __syncthreads();
    P = (P << w) | (uint64_t)d;
    need -= above;
    shift = nsh;
    if (cnt == need) break;   // the whole bucket is selected
  }

  // 3. ordered compaction: wave w owns a contiguous run of vectors; counts first, then an
  //    in-order write with wave-level prefix sums (no block barrier inside the loop).
  const int per = (n4 + NW - 1) / NW;
  const int v_lo = wave * per, v_hi = min(n4, v_lo + per);
  int gt_c = 0, eq_c = 0;
  for (int base = v_lo + lane; base < v_hi; base += kWave * kU) {
    uint32_t k[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kWave;
      if (i4 < v_hi) load_keys<CACHE>(row, kcache, i4, k[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kWave;
      if (i4 >= v_hi) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (4 * i4 + e >= n) continue;
        const uint64_t h = digit_prefix(k[u][e], shift);
        gt_c += h > P;
        eq_c += h == P;
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) { gt_c += __shfl_xor(gt_c, m); eq_c += __shfl_xor(eq_c, m); }
  if (lane == 0) { sh_gt[wave] = gt_c; sh_eq[wave] = eq_c; }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) { gt_before += sh_gt[w]; eq_before += sh_eq[w]; }
  int32_t* out = a.idx + (size_t)r * K;
  int carry_eq = eq_before;
  int carry_out = gt_before + min(eq_before, need);
  for (int i4 = v_lo + lane; i4 - lane < v_hi; i4 += kWave) {
    uint32_t k[4] = {0u, 0u, 0u, 0u};
    if (i4 < v_hi) load_keys<CACHE>(row, kcache, i4, k);
    bool gt[4], eq[4];
    int ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool valid = i4 < v_hi && 4 * i4 + e < n;
      const uint64_t h = digit_prefix(k[e], shift);
      gt[e] = valid && h > P;
      eq[e] = valid && h == P;
      ne += eq[e];
    }
    const int eq_incl = wave_incl_scan(ne);
    int eq_rank = carry_eq + eq_incl - ne;
    bool sel[4];
    int ns = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sel[e] = gt[e] || (eq[e] && eq_rank < need);
      eq_rank += eq[e];
      ns += sel[e];
    }
    const int s_incl = wave_incl_scan(ns);
    int at = carry_out + s_incl - ns;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sel[e]) {
        if (at < K) out[at] = 4 * i4 + e;
        ++at;
      }
    carry_eq += __shfl(eq_incl, kWave - 1);
    carry_out += __shfl(s_incl, kWave - 1);
  }
  if (tid == 0) a.len[r] = K;
}

// ------------------------------------------------------------ candidate filter, one row per WG
// 1. Threshold from a sample: every (n4 / 1024)-th float4 of the row (4,096 keys); T = the
//    key of rank ~1.5 K n_s / n among them to 22 leading bits, so that about 1.5 K keys of
//    the row are >= T.
// 2. One pass over the row appends every key >= T, with its position, to an LDS list
//    (wave-aggregated slots).  If the list holds fewer than K or more than kCand keys the
//    row falls back to the streaming exact selection; otherwise the top K of the row are
//    exactly the top K of the list (every key outside the list is below T).
// 3. Radix select on the list gives the K-th key and how many keys equal to it to keep; a
//    bitmap over positions then yields the kept positions in ascending order, keys equal
//    to the K-th taken lowest position first.
constexpr int kCand = 8192;
constexpr int kMaxCandRow = 4 * kCacheKeys;     // 131,072 positions: 4,096 bitmap words
constexpr int kSampleVec = 1024;

// rank-th largest (1-based) of keys[0 .. m) in LDS: returns that key and writes into *above
// the number of keys strictly greater.  Every thread of the work-group must call it.
// With stop_shift > 0 the search ends once the bits above stop_shift are known and the
// result has its low stop_shift bits cleared (a lower bound of that key; *above is then
// not meaningful).
template <int NT = kRowThreads>
__device__ uint32_t lds_select(const uint32_t* keys, int m, int rank, int* above_out,
                               uint32_t* hist, int* sh_scan, int* sh_sel, int stop_shift = 0) {
  uint32_t P = 0;        // bits of the answer above `shift`
  int shift = 32, need = rank, above_total = 0;
  while (shift > stop_shift) {
    const int w = min(kMaxDigitBits, shift);
    const int nsh = shift - w;
    const int nb = 1 << w;
    for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < m; i += NT) {
      const uint32_t k = keys[i];
      if (digit_prefix(k, shift) == P) atomicAdd(&hist[(k >> nsh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_digit<NT>(hist, nb, need, sh_sel, sh_scan);
    const int d = sh_sel[0], above = sh_sel[1];
    __syncthreads();
    P = (uint32_t)((P << w) | (uint32_t)d);
    need -= above;
    above_total += above;
    shift = nsh;
  }
  *above_out = above_total;
  return shift > 0 ? P << shift : P;
}

// Step 3 of the candidate filter, shared by the one-row kernels: the K-th key of the LDS list
// cand_key/cand_t[0 .. m) (m >= K, every key outside the list below it), then the kept
// positions in ascending order through position bitmaps of WPT words per thread.  Every
// thread of the work-group must call it.
template <int WPT>
__device__ void finish_from_candidates(const TopkLaunch& a, int r, int n, const uint32_t* cand_key,
                                       const int* cand_t, int m, uint32_t* sel_bits,
                                       uint32_t* tie_bits, uint32_t* hist, int* sh_scan,
                                       int* sh_sel) {
  const int K = a.top_k;
  const int tid = threadIdx.x;
  int above;
  const uint32_t kth = lds_select(cand_key, m, K, &above, hist, sh_scan, sh_sel);
  const int need_eq = K - above;          // keys equal to kth to keep, lowest position first
  const int nw = (n + 31) >> 5;
  for (int i = tid; i < nw; i += kRowThreads) { sel_bits[i] = 0u; tie_bits[i] = 0u; }
  __syncthreads();
  for (int i = tid; i < m; i += kRowThreads) {
    const uint32_t k = cand_key[i];
    const int t = cand_t[i];
    if (k > kth) atomicOr(&sel_bits[t >> 5], 1u << (t & 31));
    else if (k == kth) atomicOr(&tie_bits[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  // thread tid owns words [WPT * tid, WPT * tid + WPT)
  const int w0 = WPT * tid;
  int my_ties = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) my_ties += (w0 + q < nw) ? __builtin_popcount(tie_bits[w0 + q]) : 0;
  int tot;
  int tie_rank = block_exclusive_scan<kRowThreads>(my_ties, &tot, sh_scan);
  uint32_t keep[WPT];
  int my_sel = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    uint32_t sb = (w0 + q < nw) ? sel_bits[w0 + q] : 0u;
    uint32_t tb = (w0 + q < nw) ? tie_bits[w0 + q] : 0u;
    while (tb) {                                 // ties in ascending position
      const uint32_t low = tb & (0u - tb);
      if (tie_rank < need_eq) sb |= low;
      ++tie_rank;
      tb ^= low;
    }
    keep[q] = sb;
    my_sel += __builtin_popcount(sb);
  }
  int at = block_exclusive_scan<kRowThreads>(my_sel, &tot, sh_scan);
  int32_t* out = a.idx + (size_t)r * K;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    uint32_t sb = keep[q];
    while (sb) {
      const int bit = __builtin_ctz(sb);
      if (at < K) out[at] = 32 * (w0 + q) + bit;
      ++at;
      sb &= sb - 1;
    }
  }
  if (tid == 0) a.len[r] = K;
}

// Threshold of a candidate filter from a sample held NK keys per thread (every thread of a
// kRowThreads work-group calls it): the leading bits of the rank-th largest sample key,
// 11 bits at a time below the bits every sample key shares, until the sample keys >= T
// number at most lim (or 22 bits are known); the bits below are left clear.  rank must not
// exceed the sample's size.
template <int NK>
__device__ uint32_t sample_threshold(const uint32_t (&sk)[NK], int rank, int lim, uint32_t* hist,
                                     int* sh_scan, int* sh_sel, uint32_t* sh_and, uint32_t* sh_or) {
  constexpr int NW = kRowThreads / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  uint32_t av = ~0u, ov = 0u;
#pragma unroll
  for (int e = 0; e < NK; ++e) {
    av &= sk[e];
    ov |= sk[e];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    av &= (uint32_t)__shfl_xor((int)av, m);
    ov |= (uint32_t)__shfl_xor((int)ov, m);
  }
  if (lane == 0) { sh_and[wave] = av; sh_or[wave] = ov; }
  __syncthreads();
  av = ~0u; ov = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) { av &= sh_and[i]; ov |= sh_or[i]; }
  const uint32_t diff = av ^ ov;
  int shift = diff ? 32 - __builtin_clz(diff) : 0;   // bits >= shift are known
  uint32_t hm = shift >= 32 ? 0u : ~0u << shift;
  uint32_t Pk = av & hm;
  int need = rank;
  while (shift > 10) {
    const int wd = min(kMaxDigitBits, shift), nsh = shift - wd, nb = 1 << wd;
    for (int i = tid; i < nb; i += kRowThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NK; ++e)
      if ((sk[e] & hm) == Pk) atomicAdd(&hist[(sk[e] >> nsh) & (nb - 1)], 1u);
    __syncthreads();
    find_digit<kRowThreads>(hist, nb, need, sh_sel, sh_scan);
    const int d = sh_sel[0], abv = sh_sel[1], cnt = sh_sel[2];
    __syncthreads();
    Pk |= (uint32_t)d << nsh;
    hm = ~0u << nsh;
    need -= abv;
    shift = nsh;
    if (rank - need + cnt <= lim) break;   // sample keys >= T
  }
  return Pk;
}

__global__ __launch_bounds__(kRowThreads) void k_topk_cand(TopkLaunch a) {
  constexpr int NW = kRowThreads / kWave;
  __shared__ uint32_t sh_and[NW], sh_or[NW];
  __shared__ uint32_t cand_key[kCand];
  __shared__ int cand_t[kCand];
  __shared__ uint32_t sel_bits[kMaxCandRow / 32], tie_bits[kMaxCandRow / 32];
  __shared__ uint32_t hist[1 << kMaxDigitBits];
  __shared__ int sh_scan[NW];
  __shared__ int sh_sel[4];
  __shared__ int sh_count, sh_nan;

  const int r = blockIdx.x;
  int n = 0;
  if (!row_prologue(a, r, &n)) return;
  const int K = a.top_k;
  const float* row = a.scores + (size_t)r * a.ld;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int n4 = (n + 3) >> 2;

  // The first batch of the candidate pass is loaded before the threshold is known, so its
  // latency overlaps the sample selection.
  f32x4 first[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i4 = tid + u * kRowThreads;
    first[u] = i4 < n4 ? *reinterpret_cast<const f32x4*>(row + 4 * i4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // 1. threshold: the sample's rank-th key to as many leading bits as keep the list short
  uint32_t T = 0u;
  if (n > kCand) {
    const int i4 = (int)(((long long)tid * n4) / kSampleVec);   // one float4 per thread
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + 4 * i4);
    uint32_t sk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // a slot past the row's end repeats the vector's first key
      bool nn = false;
      const uint32_t k = order_key(v[e], nn);
      sk[e] = (e == 0 || 4 * i4 + e < n) ? k : sk[0];
    }
    constexpr int ns = 4 * kSampleVec;
    const float scale = (float)ns / (float)n;
    const int rank = min(ns, (int)(1.5f * (float)K * scale) + 8);
    T = sample_threshold(sk, rank, (int)(0.5f * (float)kCand * scale), hist, sh_scan, sh_sel,
                         sh_and, sh_or);
  }

  // 2. candidate list
  if (tid == 0) { sh_count = 0; sh_nan = 0; }
  __syncthreads();
  bool any_nan = false;
  // The next batch's loads are issued before the current one is filtered.
  f32x4 cur[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) cur[u] = first[u];
  for (int base = tid; base - tid < n4; base += kRowThreads * kU) {
    f32x4 nxt[kU];
    const int nb = base + kRowThreads * kU;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = nb + u * kRowThreads;
      nxt[u] = i4 < n4 ? *reinterpret_cast<const f32x4*>(row + 4 * i4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    uint32_t kv[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kRowThreads;
      if (i4 < n4) {
        const f32x4 v = cur[u];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bool nn = false;
          kv[u][e] = order_key(v[e], nn);
          any_nan |= nn && 4 * i4 + e < n;
        }
      }
    }
    int c = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kRowThreads;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += (i4 < n4 && 4 * i4 + e < n && kv[u][e] >= T) ? 1 : 0;
    }
    const int incl = wave_incl_scan(c);
    int slot = 0;
    if (lane == kWave - 1) slot = atomicAdd(&sh_count, incl);
    slot = __shfl(slot, kWave - 1) + incl - c;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i4 = base + u * kRowThreads;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i4 < n4 && 4 * i4 + e < n && kv[u][e] >= T) {
          if (slot < kCand) {
            cand_key[slot] = kv[u][e];
            cand_t[slot] = 4 * i4 + e;
          }
          ++slot;
        }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) cur[u] = nxt[u];
  }
  if (any_nan) sh_nan = 1;
  __syncthreads();
  const int m = sh_count;
  if (tid == 0 && sh_nan) raise_fault(a.fault, kFaultNan);
  if (m < K || m > kCand) {    // threshold missed: exact selection over the whole row
    __syncthreads();
    row_select_exact<false>(a, r, n, nullptr);
    return;
  }

  // 3. K-th key of the list, then the kept positions in ascending order
  finish_from_candidates<kMaxCandRow / 32 / kRowThreads>(a, r, n, cand_key, cand_t, m, sel_bits,
                                                         tie_bits, hist, sh_scan, sh_sel);
}


// ------------------------------------------------------- whole row in registers, one row per WG
// Rows up to 4,096 V positions: thread tid holds the row's float4 vectors tid + 1,024 j,
// j < V, as order-preserving keys, all loaded in one go.  The steps are those of the
// candidate filter above, but the sample and the candidate pass read these registers
// instead of the row, so the row is read from memory once and the sample selection
// overlaps the tail of its transfer.  The sample: each thread's vector tid % V (4,096 keys
// spread over the row).  A list that misses (fewer than K keys or more than kCandReg) falls
// back to the streaming exact selection.
// ADAPT (launches of at most one work-group per CU, where a row's latency is the step's):
// the threshold stops refining once the sample predicts at most half a full list, over a
// list of 8,192 keys; otherwise (many rows, throughput) 22 bits over a list of 4,096.
template <int V, bool ADAPT>
__global__ __launch_bounds__(kRowThreads) void k_topk_reg(TopkLaunch a) {
  constexpr int NW = kRowThreads / kWave;
  constexpr int kCandReg = ADAPT ? 8192 : 4096;
  __shared__ uint32_t sh_and[NW], sh_or[NW];
  constexpr int WPT = V >= 8 ? V / 8 : 1;        // bitmap words per thread (n / 32 words)
  __shared__ uint32_t cand_key[kCandReg];
  __shared__ int cand_t[kCandReg];
  __shared__ uint32_t sel_bits[WPT * kRowThreads], tie_bits[WPT * kRowThreads];
  __shared__ uint32_t hist[1 << kMaxDigitBits];
  __shared__ int sh_scan[NW];
  __shared__ int sh_sel[4];
  __shared__ int sh_count, sh_nan;

  const int r = blockIdx.x;
  int n = 0;
  if (!row_prologue(a, r, &n)) return;
  const int K = a.top_k;
  const float* row = a.scores + (size_t)r * a.ld;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int n4 = (n + 3) >> 2;
  if (tid == 0) { sh_count = 0; sh_nan = 0; }

  // Key 0 (below every order key of a number) marks NaN and the positions past n; the
  // threshold is at least 1, so they never enter the list, and a row with fewer than K other
  // keys misses and takes the exact path, which ranks NaN below -inf.
  uint32_t key[V][4];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i4 = tid + kRowThreads * j;
    const u32x4 x = i4 < n4 ? *reinterpret_cast<const u32x4*>(row + 4 * i4) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) key[j][e] = x[e];
  }
  bool any_nan = false;
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool nn = false;
      const uint32_t k = order_key(__uint_as_float(key[j][e]), nn);
      const bool valid = 4 * (tid + kRowThreads * j) + e < n;
      key[j][e] = valid ? k : 0u;
      any_nan |= nn && valid;
    }

  // 1. threshold (22 leading bits are enough; the low 10 are left clear)
  uint32_t T = 1u;
  if (n > kCandReg) {
    // n > 4,096: every thread's vector 0 is inside the row
    int js = tid % V;
    while (js > 0 && tid + kRowThreads * js >= n4) --js;
    uint32_t sk[4] = {key[0][0], key[0][1], key[0][2], key[0][3]};
#pragma unroll
    for (int j = 1; j < V; ++j)
      if (j == js) { sk[0] = key[j][0]; sk[1] = key[j][1]; sk[2] = key[j][2]; sk[3] = key[j][3]; }
    constexpr int ns = 4 * kRowThreads;
    const float scale = (float)ns / (float)n;
    const int rank = min(ns, (int)(1.5f * (float)K * scale) + 8);
    if constexpr (ADAPT) {
      T = max(1u, sample_threshold(sk, rank, (int)(0.5f * (float)kCandReg * scale), hist, sh_scan,
                                   sh_sel, sh_and, sh_or));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) cand_key[4 * tid + e] = sk[e];
      __syncthreads();
      int above;
      T = max(1u, lds_select(cand_key, ns, rank, &above, hist, sh_scan, sh_sel, 10));
    }
  }
  __syncthreads();

  // 2. candidate list from the registers
  int c = 0;
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) c += key[j][e] >= T ? 1 : 0;
  const int incl = wave_incl_scan(c);
  int slot = 0;
  if (lane == kWave - 1) slot = atomicAdd(&sh_count, incl);
  slot = __shfl(slot, kWave - 1) + incl - c;
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (key[j][e] >= T) {
        if (slot < kCandReg) {
          cand_key[slot] = key[j][e];
          cand_t[slot] = 4 * (tid + kRowThreads * j) + e;
        }
        ++slot;
      }
  if (any_nan) sh_nan = 1;
  __syncthreads();
  const int m = sh_count;
  if (tid == 0 && sh_nan) raise_fault(a.fault, kFaultNan);
  if (m < K || m > kCandReg) {    // threshold missed: exact selection over the whole row
    __syncthreads();
    row_select_exact<false>(a, r, n, nullptr);
    return;
  }
  // 3. K-th key of the list, then the kept positions in ascending order
  finish_from_candidates<WPT>(a, r, n, cand_key, cand_t, m, sel_bits, tie_bits, hist, sh_scan,
                              sh_sel);
}

// ------------------------------------------------- long rows: chunk filters, then one select
// Rows above 131,072 positions, two launches.
// 1. k_tkl_filter, one work-group per 16,384-position chunk of a row: every work-group of the
//    row takes the same threshold T from the same sample (8,192 keys for rows up to 2M
//    positions, 16,384 up to 4M, 32,768 beyond) by the same steps (T >= 1, so that NaN
//    never passes), then writes the chunk's keys >= T with their positions, in position
//    order, to the chunk's own list, and the list's length.
// 2. k_tkl_select, one work-group per row: the chunk lists taken in chunk order are the row's
//    keys >= T in position order.  With at least K and at most kLongCand of them, the top K
//    of the row are the top K of the list: thread i holds entries 16 i .. 16 i + 15 in
//    registers, radix passes below the list's common leading bits give the K-th key, and two
//    block scans place the kept positions in ascending order, keys equal to the K-th lowest
//    position first.  A list that misses takes the streaming exact selection.
constexpr int kLongEpt = 16;                          // keys per thread in both launches
constexpr int kLongChunk = kLongEpt * kRowThreads;    // 16,384 positions per filter work-group
constexpr int kLongCand = kLongEpt * kRowThreads;     // longest list the select holds
constexpr int kMaxLongChunks = kRowThreads;           // one chunk length per select thread

struct LongWs {
  int* cnt;      // [rows][chunks]              length of each chunk's list
  u32x2* list;   // [rows][chunks][kLongChunk]  (key, position), position order
};

__host__ __device__ __forceinline__ size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

__device__ __forceinline__ LongWs long_ws(void* ws, int rows, int chunks) {
  char* p = static_cast<char*>(ws);
  LongWs w;
  w.cnt = reinterpret_cast<int*>(p);
  w.list = reinterpret_cast<u32x2*>(p + round256((size_t)rows * chunks * sizeof(int)));
  return w;
}

template <int SU>
__global__ __launch_bounds__(kRowThreads) void k_tkl_filter(TopkLaunch a, int chunks) {
  constexpr int NW = kRowThreads / kWave;
  __shared__ uint32_t hist[1 << kMaxDigitBits];
  __shared__ int sh_scan[NW];
  __shared__ int sh_sel[4];
  __shared__ uint32_t sh_and[NW], sh_or[NW];
  const int r = blockIdx.x, c = blockIdx.y;
  int n = 0;
  if (row_kind(a, r, &n) != 0) return;   // the select launch writes such rows
  const int lo = c * kLongChunk, hi = min(n, lo + kLongChunk);
  if (lo >= hi) return;                  // past this row's end: the select reads no list here
  const int tid = threadIdx.x;
  const float* row = a.scores + (size_t)r * a.ld;
  const int n4 = (n + 3) >> 2;
  // The chunk's 16 keys per thread and the sample's vectors, all loads in flight at once.
  // Rows are 16-byte aligned with ld >= 4 n4, so every vector read lies inside the row.
  const int t0 = lo + kLongEpt * tid;
  f32x4 v[kLongEpt / 4];
#pragma unroll
  for (int j = 0; j < kLongEpt / 4; ++j)
    v[j] = t0 + 4 * j < hi ? *reinterpret_cast<const f32x4*>(row + t0 + 4 * j)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
  // The sample: ns = 4,096 SU keys spread over the row (SU float4 per thread).
  constexpr int ns = kRowThreads * 4 * SU;
  int si[SU];
  f32x4 sv[SU];
#pragma unroll
  for (int u = 0; u < SU; ++u) {
    const int j = tid + kRowThreads * u;
    si[u] = (int)(((long long)j * n4) / (ns / 4));
    sv[u] = *reinterpret_cast<const f32x4*>(row + 4 * si[u]);
  }
  // Sample keys in registers (NaN as key 0; a slot past the row's end repeats the first key
  // of its vector, which is inside the row).
  uint32_t sk[4 * SU];
#pragma unroll
  for (int u = 0; u < SU; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool nn = false;
      const uint32_t k = order_key(sv[u][e], nn);
      sk[4 * u + e] = (e == 0 || 4 * si[u] + e < n) ? k : sk[4 * u];
    }
  // T: until the sample keys >= T predict at most half a full list for the row; rank ~1.5 K
  // ns / n + 16, held to a predicted 0.45 of a full list and to the sample's size (a short
  // row of a long-row launch).  Every work-group of the row takes the same steps on the
  // same keys, so all find the same T.
  const float scale = (float)ns / (float)n;
  const int rank = max(1, min(ns, min((int)(1.5f * (float)a.top_k * scale) + 16,
                                      (int)(0.45f * (float)kLongCand * scale))));
  const uint32_t Pk = sample_threshold(sk, rank, (int)(0.5f * (float)kLongCand * scale), hist,
                                       sh_scan, sh_sel, sh_and, sh_or);
  const uint32_t T = max(1u, Pk);

  uint32_t key[kLongEpt], sel = 0u;
  bool nan = false;
#pragma unroll
  for (int e = 0; e < kLongEpt; ++e) {
    bool nn = false;
    key[e] = order_key(v[e >> 2][e & 3], nn);
    if (t0 + e < hi) {
      nan |= nn;
      if (key[e] >= T) sel |= 1u << e;
    }
  }
  int tot;
  int at = block_exclusive_scan<kRowThreads>(__builtin_popcount(sel), &tot, sh_scan);
  const LongWs w = long_ws(a.ws, a.s.total_q, chunks);
  u32x2* dst = w.list + ((size_t)r * chunks + c) * kLongChunk;
#pragma unroll
  for (int e = 0; e < kLongEpt; ++e)
    if ((sel >> e) & 1u) dst[at++] = u32x2{key[e], (uint32_t)(t0 + e)};
  if (tid == 0) w.cnt[(size_t)r * chunks + c] = tot;
  if (__syncthreads_or(nan) && tid == 0) raise_fault(a.fault, kFaultNan);
}

__global__ __launch_bounds__(kRowThreads) void k_tkl_select(TopkLaunch a, int chunks) {
  constexpr int NW = kRowThreads / kWave;
  __shared__ int off[kMaxLongChunks + 1];
  __shared__ __align__(16) int mark[kLongCand];
  __shared__ uint32_t hist[1 << kMaxDigitBits];
  __shared__ int sh_scan[NW];
  __shared__ int sh_sel[4];
  __shared__ uint32_t sh_and[NW], sh_or[NW];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const LongWs w = long_ws(a.ws, a.s.total_q, chunks);
  // every chunk's list length, loaded before the row is known (chunks past its end unused)
  const int cnt_ld = tid < chunks ? w.cnt[(size_t)r * chunks + tid] : 0;
  int n = 0;
  if (!row_prologue(a, r, &n)) return;
  const int K = a.top_k;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int nch = (n + kLongChunk - 1) / kLongChunk;   // <= chunks <= kMaxLongChunks
  const int mine = tid < nch ? cnt_ld : 0;
  int m;
  const int ex = block_exclusive_scan<kRowThreads>(mine, &m, sh_scan);
  if (tid < nch) off[tid] = ex;
  if (tid == nch - 1) off[nch] = ex + mine;
  __syncthreads();
  if (m < K || m > kLongCand) {   // threshold missed: exact selection over the whole row
    row_select_exact<false>(a, r, n, nullptr);
    return;
  }

  // Entries 16 tid .. 16 tid + 15 of the concatenated lists; key 0 marks an empty entry
  // (every listed key is >= T >= 1).  Entry g of chunk c's list, which starts at entry
  // off[c], sits at c * kLongChunk + (g - off[c]) = g + base(c), base(c) = c kLongChunk -
  // off[c] non-decreasing in c (a list holds at most kLongChunk keys).  mark[g] holds base(c)
  // where chunk c's (non-empty) list starts and 0 elsewhere, so an entry's base is the
  // largest mark at or before it: thread tid finds the chunk of its first entry by binary
  // search over off and carries the base forward.
  for (int i = tid; i < m; i += kRowThreads) mark[i] = 0;
  __syncthreads();
  if (tid < nch && mine > 0) mark[ex] = tid * kLongChunk - ex;
  __syncthreads();
  const int g0 = kLongEpt * tid;
  int base = 0;
  u32x4 mk[kLongEpt / 4] = {};
  if (g0 < m) {   // the last chunk c < nch with off[c] <= g0
    int l = 0, h = nch - 1;
    while (l < h) {
      const int mid = (l + h + 1) >> 1;
      if (off[mid] <= g0) l = mid; else h = mid - 1;
    }
    base = l * kLongChunk - off[l];
#pragma unroll
    for (int q = 0; q < kLongEpt / 4; ++q) mk[q] = *reinterpret_cast<const u32x4*>(mark + g0 + 4 * q);
  }
  const u32x2* lists = w.list + (size_t)r * chunks * kLongChunk;
  uint32_t key[kLongEpt];
  int pos[kLongEpt];
#pragma unroll
  for (int e = 0; e < kLongEpt; ++e) {
    const int g = g0 + e;
    const bool ok = g < m;   // entries past m read list entry 0 and are dropped
    base = max(base, (int)mk[e >> 2][e & 3]);
    const u32x2 x = lists[ok ? g + base : 0];
    key[e] = ok ? x[0] : 0u;
    pos[e] = (int)x[1];
  }

  // leading bits common to the list
  uint32_t av = ~0u, ov = 0u;
#pragma unroll
  for (int e = 0; e < kLongEpt; ++e)
    if (key[e]) { av &= key[e]; ov |= key[e]; }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    av &= (uint32_t)__shfl_xor((int)av, s);
    ov |= (uint32_t)__shfl_xor((int)ov, s);
  }
  if (lane == 0) { sh_and[wave] = av; sh_or[wave] = ov; }
  __syncthreads();
  av = ~0u; ov = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) { av &= sh_and[i]; ov |= sh_or[i]; }
  // The known leading bits as a mask and a masked key (32-bit compares on the 16 keys).
  const uint32_t diff = av ^ ov;
  int shift = diff ? 32 - __builtin_clz(diff) : 0;   // bits >= shift are known
  uint32_t hm = shift >= 32 ? 0u : ~0u << shift;
  uint32_t Pk = av & hm;
  int need = K;
  while (shift > 0) {
    const int wd = min(kMaxDigitBits, shift), nsh = shift - wd, nb = 1 << wd;
    for (int i = tid; i < nb; i += kRowThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kLongEpt; ++e)
      if (key[e] && (key[e] & hm) == Pk) atomicAdd(&hist[(key[e] >> nsh) & (nb - 1)], 1u);
    __syncthreads();
    find_digit<kRowThreads>(hist, nb, need, sh_sel, sh_scan);
    const int d = sh_sel[0], abv = sh_sel[1], cnt = sh_sel[2];
    __syncthreads();
    Pk |= (uint32_t)d << nsh;
    hm = ~0u << nsh;
    need -= abv;
    shift = nsh;
    if (cnt == need) break;   // the whole bucket is selected
  }

  // kept positions in ascending order: entries are in position order across threads
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int e = 0; e < kLongEpt; ++e)
    if (key[e]) {
      const uint32_t h = key[e] & hm;
      gt |= (h > Pk ? 1u : 0u) << e;
      eq |= (h == Pk ? 1u : 0u) << e;
    }
  int tot;
  int eq_rank = block_exclusive_scan<kRowThreads>(__builtin_popcount(eq), &tot, sh_scan);
  uint32_t sel = gt;
#pragma unroll
  for (int e = 0; e < kLongEpt; ++e)
    if ((eq >> e) & 1u) {
      if (eq_rank < need) sel |= 1u << e;
      ++eq_rank;
    }
  int at = block_exclusive_scan<kRowThreads>(__builtin_popcount(sel), &tot, sh_scan);
  int32_t* out = a.idx + (size_t)r * K;
#pragma unroll
  for (int e = 0; e < kLongEpt; ++e)
    if ((sel >> e) & 1u) {
      if (at < K) out[at] = pos[e];
      ++at;
    }
  if (tid == 0) a.len[r] = K;
}

}  // namespace

static int long_chunks(const SeqView& s) { return (s.max_seq_len + kLongChunk - 1) / kLongChunk; }

size_t topk_ws_bytes(const SeqView& s, int top_k) {
  (void)top_k;
  if (s.max_seq_len <= kMaxCandRow) return 0;
  const size_t rows = (size_t)s.total_q, chunks = (size_t)long_chunks(s);
  return round256(rows * chunks * sizeof(int)) + rows * chunks * kLongChunk * sizeof(u32x2);
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t st) {
  const SeqView& s = a.s;
  if (s.max_seq_len <= 4 * kRowThreads * 8) {
    const bool adapt = s.total_q <= 256;   // at most one work-group per CU
    if (s.max_seq_len <= 4 * kRowThreads * 4) {
      if (adapt) k_topk_reg<4, true><<<s.total_q, kRowThreads, 0, st>>>(a);
      else k_topk_reg<4, false><<<s.total_q, kRowThreads, 0, st>>>(a);
    } else {
      if (adapt) k_topk_reg<8, true><<<s.total_q, kRowThreads, 0, st>>>(a);
      else k_topk_reg<8, false><<<s.total_q, kRowThreads, 0, st>>>(a);
    }
    return hipGetLastError();
  }
  if (s.max_seq_len <= kMaxCandRow) {
    k_topk_cand<<<s.total_q, kRowThreads, 0, st>>>(a);
    return hipGetLastError();
  }
  const int chunks = long_chunks(s);
  if (chunks > kMaxLongChunks) return hipErrorInvalidValue;
  // sample float4 per thread: 2 up to 2M positions, 4 up to 4M, 8 beyond
  const dim3 grid(s.total_q, chunks);
  if (s.max_seq_len <= (2 << 20))
    k_tkl_filter<2><<<grid, kRowThreads, 0, st>>>(a, chunks);
  else if (s.max_seq_len <= (4 << 20))
    k_tkl_filter<4><<<grid, kRowThreads, 0, st>>>(a, chunks);
  else
    k_tkl_filter<8><<<grid, kRowThreads, 0, st>>>(a, chunks);
  k_tkl_select<<<s.total_q, kRowThreads, 0, st>>>(a, chunks);
  return hipGetLastError();
}

}  // namespace ml4
