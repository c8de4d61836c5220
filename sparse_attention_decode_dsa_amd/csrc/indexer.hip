// DSA indexer scores on gfx950.
//
// Pages: "vLLM 首日支持 Mistral Large 4" (best2ai.com), Implementation details › 稀疏 MLA + DSA
// indexer (FP8 indexer cache; the indexer has its own SSMax) and ROCm implementation details ›
// AITER 上的 DSA 索引器 (132-byte FP8 keys with one scale per key; paged decode scores and
// prefill scores read the FP8 keys).
//
//   s[r, t] = m_r * ks[t] * sum_h w[r,h] * qs[r,h] * ReLU(q[r,h,:] . k[t,:])
//
// The 64 x 128 x n product per query row is a real GEMM even for one decode token, so it
// runs on the matrix cores: heads on the MFMA M axis (16 per tile), keys on N, the 128 key
// dims on K.  It uses v_mfma_f32_16x16x32_f16: every e4m3 code converts exactly to fp16, so
// products are exact and the four K=32 steps accumulate in fp32.  (The fp8 form
// v_mfma_f32_16x16x128_f8f6f4 drops low-order bits of small products inside its 128-term sum
// -- measured up to 1.3e-5 of sum |q_d k_d| on gfx950 against 6.5e-8 for the 16-bit forms --
// which moves keys across the top-k boundary.)
//
// A work-group owns one request's run of up to 4 query rows and a chunk of its keys.  Key
// rows stream from HBM in steps of 64 keys (4 rows per work-group) or 128 keys (1 or 2
// rows: half as many barriers per key, measured 9 % faster for a 1M-key single-row decode,
// 3 % for 2-row verify and 1 % for 8 x 32k decode, while 4 rows lose 5 % to register
// pressure): each thread loads 32 bytes of a row
// (of two rows, 64 keys apart, in 128-key steps), decodes them to fp16 and writes them to
// a double-buffered LDS tile, so a key is fetched and decoded once for all rows.  Each wave
// owns one query row (its 64 x 128 query stays in registers) and 16-key sub-tiles of the
// step; the weighted-ReLU head reduction runs in-lane over the 4 heads a lane holds per
// tile, then across the 4 lane groups.
#include "ml4_device.h"

namespace ml4 {

namespace {

constexpr int kIdxRow = 132;
// Keys per staging step for R query rows per work-group.
template <int R>
constexpr int step_keys() { return R == 4 ? 64 : 128; }
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kKeyStride = 136;   // fp16 per key row in LDS (128 + 8): conflict-free b128 reads

// v[s] summed over the four 16-lane groups, delivered to lane group s (same column):
// permlane32_swap pairs groups g and g ^ 2, permlane16_swap then pairs g and g ^ 1.
__device__ __forceinline__ float sum_over_lane_groups(const float (&v)[4]) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]),
                                                  false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]),
                                                  false, false);
  const float xs = __uint_as_float(x[0]) + __uint_as_float(x[1]);   // groups 0,1: v0; 2,3: v2
  const float ys = __uint_as_float(y[0]) + __uint_as_float(y[1]);   // groups 0,1: v1; 2,3: v3
  const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(xs), __float_as_uint(ys),
                                                  false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

constexpr int kMaxKeysPerWg = 4096;

// R = query rows per work-group (1, 2 or 4), HT = 16-head tiles (n_heads / 16).
template <int R, int HT>
__global__ __launch_bounds__(kThreads)
void k_indexer_fp8(IndexerLaunch a, int groups_per_seq, int keys_per_wg) {
  constexpr int kStepKeys = step_keys<R>();
  constexpr int kHalves = kStepKeys / 64;        // staged keys per thread and step
  __shared__ __attribute__((aligned(16))) _Float16 ktile[2][kStepKeys * kKeyStride];
  __shared__ float kscale[2][kStepKeys];
  __shared__ int kok[2][kStepKeys / 16];
  __shared__ int blk_sh[kMaxKeysPerWg / 16];   // block of each 16-key group of the chunk

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int g16 = lane >> 4;
  const int c16 = lane & 15;
  const SeqView& s = a.s;
  const int b = blockIdx.y / groups_per_seq;
  const int grp = blockIdx.y - b * groups_per_seq;
  const int q0 = s.q_start[b];
  const int nq = s.q_start[b + 1] - q0;
  const int row0 = q0 + grp * R;
  const int nrows = min(R, nq - grp * R);
  if (nrows <= 0) return;
  const int seq_len = s.seq_lens[b];
  const int k_lo = blockIdx.x * keys_per_wg;
  const int k_hi = min(k_lo + keys_per_wg, s.max_seq_len);
  if (k_lo >= k_hi) return;

  // Positions of the work-group's rows; the keys it must score end at the largest.
  int pmax = -1;
  for (int j = 0; j < nrows; ++j) {
    const int p = s.q_pos[row0 + j];
    if (p >= 0 && p < seq_len && p < s.max_seq_len) pmax = max(pmax, p);
  }
  // This wave's row: wave % R (waves beyond nrows mirror row 0 but write nothing).
  const int jr = wave % R;
  const bool row_live = jr < nrows;
  const int row = row0 + (row_live ? jr : 0);
  int pos = s.q_pos[row];
  if (pos < 0 || pos >= seq_len || pos >= s.max_seq_len) {
    if (row_live && blockIdx.x == 0 && lane == 0) raise_fault(a.fault, 1u << 3);
    pos = -1;
  }
  // The 4/R waves of a row split the step's four 16-key sub-tiles: wave / R, + 4 / R, ...
  constexpr int kSubPerWave = (kStepKeys / 16) * R / kWaves;
  const int sub0 = wave / R;

  const int32_t* bt = s.block_table + (size_t)b * s.mbps;
  const int k_end = min(k_hi, pmax + 1);          // keys scored: k_lo .. k_end - 1
  // Block of every 16-key group up to k_end (16 consecutive keys share a block since the
  // block size is a power of two >= 16); -1 marks a block id outside the pool.
  for (int gi = tid; gi * 16 < k_end - k_lo; gi += kThreads) {
    const int blk = bt[(k_lo + 16 * gi) >> s.lbs];
    if ((unsigned)blk >= (unsigned long long)a.num_blocks) {
      raise_fault(a.fault, 1u << 0);
      blk_sh[gi] = -1;
    } else {
      blk_sh[gi] = blk;
    }
  }

  // Query fragments (A operand: head on M, dims on K).  Lane group g holds dims 32g .. 32g+31
  // as four K=32 chunks; the key side uses the same split, so the dims pair up.
  f16x8 qa[HT][4];
  float wq[HT][4];
  const uint8_t* qbase = static_cast<const uint8_t*>(a.q);
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint8_t* qp = qbase + ((size_t)row * a.n_heads + ht * 16 + c16) * 128 + 32 * g16;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(qp);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(qp + 16);
    const uint32_t w8[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x4 lo = e4m3x4_to_f16(w8[2 * c]);
      const f16x4 hi = e4m3x4_to_f16(w8[2 * c + 1]);
      qa[ht][c] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t o = (size_t)row * a.n_heads + ht * 16 + 4 * g16 + i;
      wq[ht][i] = a.w[o] * (a.q_scale ? a.q_scale[o] : 1.0f);
    }
  }
  const float mrow = ssmax_mult(a.ssmax_s, max(pos, 0));

  const uint8_t* pool = static_cast<const uint8_t*>(a.pool);
  const int bs_mask = (1 << s.lbs) - 1;
  const float ninf = -__builtin_inff();

  // Keys past every row's position only get -inf.
  for (int t = max(k_lo, k_end) + tid; t < k_hi; t += kThreads)
    for (int j = 0; j < nrows; ++j) a.scores[(size_t)(row0 + j) * a.ld + t] = ninf;
  const int nsteps = (k_end - k_lo + kStepKeys - 1) / kStepKeys;
  if (nsteps <= 0) return;
  __syncthreads();   // blk_sh

  // Staging: thread -> (keys kk + 64 j, quarter qq = tid % 4) of a step, kk = tid / 4.
  // Two register sets keep the loads of two steps in flight.
  const int kk = tid >> 2, qq = tid & 3;
  struct Half {
    u32x4 lo, hi;
    float scale;
    int ok;
  };
  struct Stage {
    Half h[kHalves];
  };
  auto load_half = [&](Half& S, int t) {
    S.lo = u32x4{0, 0, 0, 0};
    S.hi = u32x4{0, 0, 0, 0};
    S.scale = 0.f;
    S.ok = 0;
    if (t >= k_end) return;      // past every row: nothing is read
    const int blk = blk_sh[(t - k_lo) >> 4];
    if (blk < 0) return;
    const uint8_t* rp = pool + (((int64_t)blk << s.lbs) + (t & bs_mask)) * kIdxRow;
    const u32x4a4 v0 = *reinterpret_cast<const u32x4a4*>(rp + 32 * qq);
    const u32x4a4 v1 = *reinterpret_cast<const u32x4a4*>(rp + 32 * qq + 16);
    S.lo = u32x4{v0[0], v0[1], v0[2], v0[3]};
    S.hi = u32x4{v1[0], v1[1], v1[2], v1[3]};
    if (qq == 0) S.scale = *reinterpret_cast<const float*>(rp + 128);
    S.ok = 1;
  };
  auto load_step = [&](Stage& S, int t0) {
#pragma unroll
    for (int j = 0; j < kHalves; ++j) load_half(S.h[j], t0 + 64 * j + kk);
  };
  auto store_half = [&](const Half& S, int buf, int key) {
    _Float16* dst = &ktile[buf][key * kKeyStride + 32 * qq];
    const uint32_t w8[8] = {S.lo[0], S.lo[1], S.lo[2], S.lo[3],
                            S.hi[0], S.hi[1], S.hi[2], S.hi[3]};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x4 lo = e4m3x4_to_f16(w8[2 * c]);
      const f16x4 hi = e4m3x4_to_f16(w8[2 * c + 1]);
      *reinterpret_cast<f16x8*>(dst + 8 * c) =
          f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    if (qq == 0) kscale[buf][key] = S.scale;
    if (qq == 0 && (key & 15) == 0) kok[buf][key >> 4] = S.ok;
  };
  auto store_step = [&](const Stage& S, int buf) {
#pragma unroll
    for (int j = 0; j < kHalves; ++j) store_half(S.h[j], buf, 64 * j + kk);
  };
  // Scores of one step for this wave's row.  Each lane accumulates, per sub-tile, the
  // weighted ReLU over the 4 heads of each head tile it holds; a cross-lane transpose-sum
  // (two permlane32 and one permlane16 swap) per four sub-tiles then leaves sub-tile g's
  // totals in lane group g, so the row's results leave in one store per four sub-tiles.  K fragments of the next sub-tile are
  // read while the current one multiplies.
  auto compute_step = [&](int st, int buf) {
    const int t0 = k_lo + st * kStepKeys;
    float part[kSubPerWave];
#pragma unroll
    for (int i = 0; i < kSubPerWave; ++i) part[i] = 0.f;
    f16x8 kb[2][4];
    auto read_frags = [&](f16x8 (&dst)[4], int sub) {
      const _Float16* krow = &ktile[buf][(16 * sub + c16) * kKeyStride + 32 * g16];
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[c] = *reinterpret_cast<const f16x8*>(krow + 8 * c);
    };
    read_frags(kb[0], sub0);
#pragma unroll
    for (int si = 0; si < kSubPerWave; ++si) {
      if (si + 1 < kSubPerWave) read_frags(kb[(si + 1) & 1], sub0 + (si + 1) * (kWaves / R));
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4 d{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) d = mfma_f16(qa[ht][c], kb[si & 1][c], d);
#pragma unroll
        for (int i = 0; i < 4; ++i) part[si] = fmaf(wq[ht][i], relu_bits(d[i]), part[si]);
      }
    }
#pragma unroll
    for (int h = 0; h < (kSubPerWave + 3) / 4; ++h) {
      float p4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p4[j] = 4 * h + j < kSubPerWave ? part[4 * h + j] : 0.f;
      const float tot = sum_over_lane_groups(p4);
      const int sl = 4 * h + g16;                    // this lane group's sub-tile of the wave
      const int sub = sub0 + sl * (kWaves / R);
      const int t = t0 + 16 * sub + c16;
      if (row_live && sl < kSubPerWave && t < k_hi) {
        const bool ok = t < k_end && t <= pos && kok[buf][sub] != 0;
        a.scores[(size_t)row * a.ld + t] = ok ? tot * kscale[buf][16 * sub + c16] * mrow : ninf;
      }
    }
  };

  Stage SA, SB;
  load_step(SA, k_lo);
  if (nsteps > 1) load_step(SB, k_lo + kStepKeys);
  store_step(SA, 0);
  __syncthreads();
  // Step st computes buffer st & 1, issues the loads of step st + 2 and stages step st + 1
  // (loaded during step st - 1) into the other buffer.
  for (int st = 0; st < nsteps; st += 2) {
    if (st + 2 < nsteps) load_step(SA, k_lo + (st + 2) * kStepKeys);
    compute_step(st, 0);
    if (st + 1 < nsteps) store_step(SB, 1);
    __syncthreads();
    if (st + 1 >= nsteps) break;
    if (st + 3 < nsteps) load_step(SB, k_lo + (st + 3) * kStepKeys);
    compute_step(st + 1, 1);
    if (st + 2 < nsteps) store_step(SA, 0);
    __syncthreads();
  }
}

// One query row per work-group (decode): with a single row there is nothing to share, so
// each key is decoded once in any case and the LDS staging, with its barrier per step, is
// pure latency.  Here every wave scores its own 64-key blocks (w, w + 4, ... of the chunk)
// straight from HBM: lane (g, c) loads the 32 bytes of key c that hold dims 32 g .. 32 g + 31
// -- exactly its B-operand fragment -- decodes them in registers and multiplies; the next
// block's loads are in flight meanwhile.  No barrier after the block table.  The arithmetic
// (fragment dims, MFMA order, head reduction, transpose-sum) is that of k_indexer_fp8, so
// the scores are bit-identical.
template <int HT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_indexer_row(IndexerLaunch a, int keys_per_wg) {
  __shared__ int blk_sh[kMaxKeysPerWg / 16];   // block of each 16-key group of the chunk

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int g16 = lane >> 4;
  const int c16 = lane & 15;
  const SeqView& s = a.s;
  const int b = blockIdx.y;
  const int row = s.q_start[b];
  if (s.q_start[b + 1] - row <= 0) return;
  const int seq_len = s.seq_lens[b];
  const int k_lo = blockIdx.x * keys_per_wg;
  const int k_hi = min(k_lo + keys_per_wg, s.max_seq_len);
  if (k_lo >= k_hi) return;
  int pos = s.q_pos[row];
  if (pos < 0 || pos >= seq_len || pos >= s.max_seq_len) {
    if (blockIdx.x == 0 && tid == 0) raise_fault(a.fault, 1u << 3);
    pos = -1;
  }
  const int32_t* bt = s.block_table + (size_t)b * s.mbps;
  const int k_end = min(k_hi, pos + 1);          // keys scored: k_lo .. k_end - 1
  for (int gi = tid; gi * 16 < k_end - k_lo; gi += kThreads) {
    const int blk = bt[(k_lo + 16 * gi) >> s.lbs];
    if ((unsigned)blk >= (unsigned long long)a.num_blocks) {
      raise_fault(a.fault, 1u << 0);
      blk_sh[gi] = -1;
    } else {
      blk_sh[gi] = blk;
    }
  }

  f16x8 qa[HT][4];
  float wq[HT][4];
  const uint8_t* qbase = static_cast<const uint8_t*>(a.q);
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint8_t* qp = qbase + ((size_t)row * a.n_heads + ht * 16 + c16) * 128 + 32 * g16;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(qp);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(qp + 16);
    const uint32_t w8[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x4 lo = e4m3x4_to_f16(w8[2 * c]);
      const f16x4 hi = e4m3x4_to_f16(w8[2 * c + 1]);
      qa[ht][c] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t o = (size_t)row * a.n_heads + ht * 16 + 4 * g16 + i;
      wq[ht][i] = a.w[o] * (a.q_scale ? a.q_scale[o] : 1.0f);
    }
  }
  const float mrow = ssmax_mult(a.ssmax_s, max(pos, 0));
  const uint8_t* pool = static_cast<const uint8_t*>(a.pool);
  const int bs_mask = (1 << s.lbs) - 1;
  const float ninf = -__builtin_inff();
  float* srow = a.scores + (size_t)row * a.ld;

  for (int t = max(k_lo, k_end) + tid; t < k_hi; t += kThreads) srow[t] = ninf;
  const int nblk = (k_end - k_lo + 63) / 64;     // 64-key blocks holding scored keys
  __syncthreads();   // blk_sh
  if (wave >= nblk) return;

  // Sub-tile j of block m: keys k_lo + 64 (wave + 4 m) + 16 j + c; lane (g, c) holds key c.
  struct Frag {
    u32x4 lo, hi;
    float scale;
    int ok;
  };
  auto load = [&](Frag& F, int m, int j) {
    F.lo = u32x4{0, 0, 0, 0};
    F.hi = u32x4{0, 0, 0, 0};
    F.scale = 0.f;
    F.ok = 0;
    const int t = k_lo + 64 * (wave + 4 * m) + 16 * j + c16;
    if (wave + 4 * m >= nblk || t >= k_end) return;
    const int blk = blk_sh[(t - k_lo) >> 4];
    if (blk < 0) return;
    const uint8_t* rp = pool + (((int64_t)blk << s.lbs) + (t & bs_mask)) * kIdxRow;
    const u32x4a4 v0 = *reinterpret_cast<const u32x4a4*>(rp + 32 * g16);
    const u32x4a4 v1 = *reinterpret_cast<const u32x4a4*>(rp + 32 * g16 + 16);
    F.lo = u32x4{v0[0], v0[1], v0[2], v0[3]};
    F.hi = u32x4{v1[0], v1[1], v1[2], v1[3]};
    F.scale = *reinterpret_cast<const float*>(rp + 128);
    F.ok = 1;
  };
  Frag f0, f1, f2, f3;
  load(f0, 0, 0);
  load(f1, 0, 1);
  load(f2, 0, 2);
  load(f3, 0, 3);
  for (int m = 0; wave + 4 * m < nblk; ++m) {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    float keep_scale = 0.f;    // of sub-tile g16's key c16 (this lane's column after the sum)
    int keep_ok = 0;
    auto sub = [&](Frag& F, int j) {
      const uint32_t w8[8] = {F.lo[0], F.lo[1], F.lo[2], F.lo[3],
                              F.hi[0], F.hi[1], F.hi[2], F.hi[3]};
      if (g16 == j) {
        keep_scale = F.scale;
        keep_ok = F.ok;
      }
      f16x8 kb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f16x4 lo = e4m3x4_to_f16(w8[2 * c]);
        const f16x4 hi = e4m3x4_to_f16(w8[2 * c + 1]);
        kb[c] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      load(F, m + 1, j);       // the next block's sub-tile j, in flight while this block runs
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4 d{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) d = mfma_f16(qa[ht][c], kb[c], d);
#pragma unroll
        for (int i = 0; i < 4; ++i) part[j] = fmaf(wq[ht][i], relu_bits(d[i]), part[j]);
      }
    };
    sub(f0, 0);
    sub(f1, 1);
    sub(f2, 2);
    sub(f3, 3);
    const float tot = sum_over_lane_groups(part);
    const int t = k_lo + 64 * (wave + 4 * m) + 16 * g16 + c16;
    if (t < k_hi) srow[t] = (t < k_end && keep_ok) ? tot * keep_scale * mrow : ninf;
  }
}

// fp32 format: 128 x fp32 per key, no key scale, fp32 queries.  One thread per key, the
// row's queries in LDS.
__global__ __launch_bounds__(256) void k_indexer_f32(IndexerLaunch a) {
  __shared__ float qsh[64 * 128];
  __shared__ float wsh[64];
  const SeqView& s = a.s;
  const int r = blockIdx.y;
  const int b = request_of(s.q_start, s.batch, r);
  const int H = a.n_heads;
  const float* q = static_cast<const float*>(a.q) + (size_t)r * H * 128;
  for (int i = threadIdx.x; i < H * 128; i += 256) qsh[i] = q[i];
  for (int h = threadIdx.x; h < H; h += 256)
    wsh[h] = a.w[(size_t)r * H + h] * (a.q_scale ? a.q_scale[(size_t)r * H + h] : 1.0f);
  __syncthreads();
  int p = s.q_pos[r];
  if (p < 0 || p >= s.seq_lens[b] || p >= s.max_seq_len) {
    if (blockIdx.x == 0 && threadIdx.x == 0) raise_fault(a.fault, 1u << 3);
    p = -1;
  }
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= s.max_seq_len) return;
  float* out = a.scores + (size_t)r * a.ld + t;
  if (t > p) {
    *out = -__builtin_inff();
    return;
  }
  const int blk = s.block_table[(size_t)b * s.mbps + (t >> s.lbs)];
  if ((unsigned)blk >= (unsigned long long)a.num_blocks) {
    raise_fault(a.fault, 1u << 0);
    *out = -__builtin_inff();
    return;
  }
  const float* k = static_cast<const float*>(a.pool) +
                   (((int64_t)blk << s.lbs) + (t & ((1 << s.lbs) - 1))) * 128;
  float kr[128];
#pragma unroll
  for (int i = 0; i < 128; i += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(k + i);
    kr[i] = v[0]; kr[i + 1] = v[1]; kr[i + 2] = v[2]; kr[i + 3] = v[3];
  }
  float acc = 0.f;
  for (int h = 0; h < H; ++h) {
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 128; ++i) d = fmaf(qsh[h * 128 + i], kr[i], d);
    acc += wsh[h] * fmaxf(d, 0.f);
  }
  *out = acc * ssmax_mult(a.ssmax_s, p);
}

template <int R>
hipError_t dispatch_heads(const IndexerLaunch& a, dim3 grid, int gps, int kpw, hipStream_t st) {
  if constexpr (R == 1) {
    switch (a.n_heads / 16) {
      case 1: k_indexer_row<1><<<grid, kThreads, 0, st>>>(a, kpw); break;
      case 2: k_indexer_row<2><<<grid, kThreads, 0, st>>>(a, kpw); break;
      case 3: k_indexer_row<3><<<grid, kThreads, 0, st>>>(a, kpw); break;
      case 4: k_indexer_row<4><<<grid, kThreads, 0, st>>>(a, kpw); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (a.n_heads / 16) {
    case 1: k_indexer_fp8<R, 1><<<grid, kThreads, 0, st>>>(a, gps, kpw); break;
    case 2: k_indexer_fp8<R, 2><<<grid, kThreads, 0, st>>>(a, gps, kpw); break;
    case 3: k_indexer_fp8<R, 3><<<grid, kThreads, 0, st>>>(a, gps, kpw); break;
    case 4: k_indexer_fp8<R, 4><<<grid, kThreads, 0, st>>>(a, gps, kpw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t st) {
  const SeqView& s = a.s;
  if (!a.fp8) {
    dim3 grid((s.max_seq_len + 255) / 256, s.total_q);
    k_indexer_f32<<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  const int R = s.max_q_per_seq <= 1 ? 1 : (s.max_q_per_seq <= 2 ? 2 : 4);
  const int gps = (s.max_q_per_seq + R - 1) / R;
  const long long groups = (long long)s.batch * gps;
  // Keys per work-group: long chunks amortise loading the queries; shrink them until the
  // grid covers the 256 CUs several times over.  Single-row decode streams HBM and wants
  // fewer, longer chunks (512 work-groups: 8 x 32k rows 17.1 -> 15.5 us); rows sharing
  // each key load run on the matrix cores and want more (2,048: 4-row verify 233 -> 222 us).
  const long long target = R == 1 ? 512 : 2048;
  int kpw = kMaxKeysPerWg;
  while (kpw > 256 && groups * ((s.max_seq_len + kpw - 1) / kpw) < target) kpw >>= 1;
  dim3 grid((s.max_seq_len + kpw - 1) / kpw, (unsigned)groups);
  switch (R) {
    case 1: return dispatch_heads<1>(a, grid, gps, kpw, st);
    case 2: return dispatch_heads<2>(a, grid, gps, kpw, st);
    default: return dispatch_heads<4>(a, grid, gps, kpw, st);
  }
}

}  // namespace ml4
