// Sparse MLA attention over the selected latent rows, on gfx950.
//
// Pages: "vLLM 首日支持 Mistral Large 4" (best2ai.com): Highlights (MLA with KV LoRA rank 512,
// RoPE dim 64, top-2048 keys per query); Implementation details › 稀疏 MLA + DSA indexer
// (sparse MLA over the fp8_ds_mla latent cache) and › NoPE、SSMax 和 LeRoPE (NoPE is MLA with
// RoPE dim 0 on the same kernel and layout; SSMax logit scaling); › 跨层 KV 共享 (consumers
// read the target layer's cache); ROCm implementation details › AITER 上的稀疏 MLA (top-k
// positions become global cache slots, one entry per query token); Long context › DCP
// (partial attentions merged through their log-sum-exp).
//
// One work-group = one query row x up to 128 heads x a contiguous range of its selected
// keys, 8 waves.  Per 32-key tile:
//   gather  the selected 656-byte rows (slot = block_table[t / bs] * bs + t % bs) straight
//           into a three-tile LDS ring with 16-byte global->LDS transfers, issued two tiles
//           ahead of the math; the rows keep the cache layout and are never rewritten;
//   QK      S^T = K . Q^T with keys on M and heads on N, on v_mfma_f32_16x16x32_bf16 with
//           the bf16 query as given: latent K fragments are read as e4m3 and decoded exactly
//           to bf16 in registers (every e4m3 value is a bf16 value, and a product of two bf16
//           values is exact in the fp32 accumulator); each wave contracts one half of the
//           latent dims (its two 128-dim scale blocks, each summed on its own and multiplied
//           by its key's scale in fp32) and half of the RoPE dims, for 32 heads; the partner
//           wave's half arrives through LDS (a NoPE layer never touches the RoPE bytes);
//   softmax online, base 2, per head = per lane column; the running maximum only moves when
//           a tile exceeds it by more than 2^8, so the accumulator is rarely rescaled; the
//           logit scale rides in the exponent's fma, and keys without a slot are masked only
//           in tiles whose validity mask (one ballot per tile, built with the slot table)
//           says they hold one;
//   PV      O^T = V^T . P^T on v_mfma_f32_16x16x32_f16 with latent columns on M, heads on
//           N, over the wave's 256 latent dims: V^T fragments come from the e4m3 rows through
//           ds_read_b64_tr_b8 and are decoded in registers, P^T comes from the QK
//           accumulators in place (the key order of both operands is the same permutation),
//           and the per-128 scale of V is folded into P per column block.  fp16 keeps 11
//           significant bits of P, which bounds the output error by 2^-11 * sum_t p_t |c_t|
//           even when SSMax makes the softmax peaked.
// One work-group barrier per tile: after QK the waves wait for the next tile's transfers,
// so the barrier that publishes the partial S also publishes the next tile.  With at most
// 64 heads (the model's own head count, or a tensor-parallel share) half of those waves
// would idle; there two wave groups take alternate tiles of the row instead, each with its
// own softmax state, merged through LDS at the end (two barriers per step of two tiles).
// A row's selected keys may be split across work-groups; the partial results are merged by
// their log-sum-exp in a second kernel.
#include "ml4_device.h"

namespace ml4 {

namespace {

constexpr int kTK = 32;            // keys per tile
constexpr int kQRS = 80;           // bf16 stride of a head's RoPE query in LDS (64 + 16:
                                   // conflict-free 16-byte reads)
constexpr float kRescaleSlack = 8.0f;
constexpr float kMaxVScale = 128.0f;   // 2^8 * 128 * 448 stays inside fp16 after P * scale
constexpr uint32_t kFaultBlock = 1u << 0;
constexpr uint32_t kFaultTopk = 1u << 1;
constexpr uint32_t kFaultQpos = 1u << 3;
constexpr uint32_t kFaultRange = 1u << 4;



// Source of the gather for masked keys and for lanes past the end of a tile.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[16];
constexpr int kMaxSplitKeys = 2048;   // top_k <= 2048
constexpr int kMlaThreads = 512;
constexpr int kMlaWaves = 8;
constexpr int kHeadsPerWg = 128;

// Waits until at most n of this wave's vector-memory operations are outstanding (vmcnt).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14]; expcnt (bits 6:4) and lgkmcnt
  // (bits 11:8) left at their maxima so only vmcnt is waited on.
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at
// lds + 16 l (lds is wave-uniform, passed in M0).  Written as inline asm so that the
// compiler does not see an LDS write of unknown address in flight: it would otherwise wait
// for every outstanding transfer before the next LDS read, which defeats the prefetch.
// Completion is tracked explicitly with wait_vmcnt<> followed by a work-group barrier.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// Sum / maximum over the four 16-lane groups, in every lane of a column: permlane32_swap
// pairs lane groups g and g ^ 2, permlane16_swap then pairs g and g ^ 1.
__device__ __forceinline__ float max_over_lane_groups(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
}
__device__ __forceinline__ float sum_over_lane_groups(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

// LDS layout of one work-group (bytes).  The gather ring holds NBLK 1-KB blocks per tile
// (one transfer instruction each); instructions past the tile write a junk block.  The
// tile's rows sit at a stride of RS = 16 NCH bytes with the cache row's own layout, and the
// matrix-core operands are read from there directly.
//   FMT kFmtFp8:  fp8_ds_mla rows, [512 e4m3][4 x fp32 scale][64 x bf16 RoPE] = 656 B;
//   FMT kFmtBf16: bf16 rows, [512 x bf16][64 x bf16 RoPE] = 1,152 B (a two-tile ring);
//   FMT kFmtE4m3: plain E4M3 rows, [512 x e4m3][64 x e4m3 RoPE] = 576 B, one per-tensor scale.
//                 A NoPE layer gathers 33 chunks (528 B) per row: the padding chunk (RoPE
//                 bytes, never read) keeps rows off a 512-B LDS stride.
constexpr int kFmtFp8 = 0, kFmtBf16 = 1, kFmtE4m3 = 2;

template <int ROPE, int FMT, bool TG = false>
struct MlaGeom {
  static constexpr int ROW_BYTES =                                  // cache row stride
      FMT == kFmtFp8 ? 656 : FMT == kFmtBf16 ? 1152 : 576;
  static constexpr int ROPE_OFF = FMT == kFmtFp8 ? 528 : FMT == kFmtBf16 ? 1024 : 512;
  static constexpr int NCH =                                        // 16-B chunks read per row
      ROPE ? ROW_BYTES / 16 : FMT == kFmtE4m3 ? 33 : ROPE_OFF / 16;
  // One barrier per tile (fp8_ds_mla and plain E4M3 rows): a three-tile ring and two
  // partial-S buffers, so that the barrier after QK also publishes the next tile.  The bf16 rows do not fit that and
  // keep two barriers per tile over a two-tile ring.
  static constexpr bool ONEBAR = FMT != kFmtBf16;
  // Two wave groups (at most 64 heads): four tile slots (two steps of two tiles), one
  // exchange buffer.
  static constexpr int NSTAGE = TG ? 4 : ONEBAR ? 3 : 2;
  static constexpr int XS_BUFS = TG ? 1 : ONEBAR ? 2 : 1;
  static constexpr int RS = 16 * NCH;                   // bytes per gathered row
  static constexpr int RAW = kTK * NCH;                 // chunks per tile
  static constexpr int NBLK = (RAW + kWave - 1) / kWave;
  static constexpr int PER_WAVE = (NBLK + kMlaWaves - 1) / kMlaWaves;
  static constexpr int STAGE = NBLK * 1024;
  static constexpr int OFF_JUNK = NSTAGE * STAGE;
  static constexpr int OFF_XS = OFF_JUNK + 1024;                      // [8][4][64] f32x4
  static constexpr int XS_WORDS = kMlaWaves * 4 * kWave;            // f32x4 per buffer
  static constexpr int OFF_QR = OFF_XS + XS_BUFS * XS_WORDS * 16;    // [128][kQRS] bf16
  static constexpr int OFF_SLOT = OFF_QR + (ROPE && FMT != kFmtE4m3 ? kHeadsPerWg * kQRS * 2 : 0);
  static constexpr int OFF_MASK = OFF_SLOT + kMaxSplitKeys * 4;        // [tiles] u32
  static constexpr int BYTES = OFF_MASK + (kMaxSplitKeys / kTK) * 4;
};
static_assert(MlaGeom<64, kFmtFp8>::BYTES <= 160 * 1024, "LDS budget");
static_assert(MlaGeom<64, kFmtFp8, true>::BYTES <= 160 * 1024, "LDS budget");
static_assert(MlaGeom<64, kFmtE4m3, true>::BYTES <= 160 * 1024, "LDS budget");
static_assert(MlaGeom<64, kFmtBf16>::BYTES <= 160 * 1024, "LDS budget");
static_assert(MlaGeom<0, kFmtFp8>::RS == 528 && MlaGeom<64, kFmtFp8>::RS == 656, "rows");
static_assert(MlaGeom<0, kFmtBf16>::RS == 1024 && MlaGeom<64, kFmtBf16>::RS == 1152, "rows");
static_assert(MlaGeom<64, kFmtE4m3>::BYTES <= 160 * 1024, "LDS budget");
static_assert(MlaGeom<0, kFmtE4m3>::RS == 528 && MlaGeom<64, kFmtE4m3>::RS == 576, "rows");

// Work split inside a work-group of 8 waves (one query row, up to 128 heads): wave w owns
// head group hg = w >> 1 (32 heads = two 16-head MFMA tiles) and dim half dh = w & 1
// (latent dims 256 dh .. 256 dh + 255, RoPE dims 32 dh .. 32 dh + 31).  Every K or V
// fragment read from LDS feeds two MFMAs.  Per wave the latent query takes 64 registers and
// the output accumulator 128; the RoPE query is read from LDS per tile.

constexpr int kQkAhead = 2;   // bf16 K fragments in flight ahead of the MFMAs

// Scale offset of an fp8_ds_mla row.
constexpr int kScaleOff = 512;

// Query fragments per head tile: bf16 as given for the fp8_ds_mla and the bf16 rows (8 x 32
// dims each), E4M3 codes for the plain E4M3 rows (two 128-dim latent fragments and one
// RoPE fragment, 32 bytes per lane each).
template <int FMT> struct QFrag { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct QFrag<kFmtE4m3> { typedef i32x8 type; static constexpr int N = 3; };

// Eight bf16 values (four per 64-bit half) -> fp16, exactly for |x| in [2^-14, 65504]
// (8 significant bits fit in 11): the bf16 bits shifted up are the binary32 value, and the
// truncating pack loses nothing.
__device__ __forceinline__ f16x8 bf16x8_to_f16(const s16x4& lo, const s16x4& hi) {
  f16x8 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const s16x4& v = h ? hi : lo;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float a = __uint_as_float((uint32_t)(uint16_t)v[e] << 16);
      const float b = __uint_as_float((uint32_t)(uint16_t)v[e + 1] << 16);
      const auto pk = __builtin_amdgcn_cvt_pkrtz(a, b);
      r[4 * h + e] = pk[0];
      r[4 * h + e + 1] = pk[1];
    }
  }
  return r;
}

// Partial S^T of key sub-tile kt over this wave's dims for the bf16 and plain E4M3 rows:
// rows = keys 16 kt + 4 g + j (+ the interleave of the row layout), columns = heads.
template <int ROPE, int FMT, int DH>
__device__ __forceinline__ void qk_part(const unsigned char* raw, const __bf16* qr_lane,
                                        const typename QFrag<FMT>::type (&qb)[2][QFrag<FMT>::N],
                                        int kt, f32x4 (&sk)[2], int g16, int c16) {
  using G = MlaGeom<ROPE, FMT>;
  constexpr int RS = G::RS;
  if constexpr (FMT == kFmtE4m3) {
    // FP8 x FP8 on v_mfma_scale_f32_16x16x128_f8f6f4: lane (g, i) supplies key 16 kt + i,
    // bytes 32 g .. 32 g + 31 of each 128-dim chunk.  Half 0 also takes the 64 RoPE dims
    // (lane groups 2, 3 of that fragment are zero on both sides).  The logit scale
    // (kv_scale * q_scale * sigma) is applied to the sum by the caller.
    const unsigned char* krow = raw + (kt * 16 + c16) * RS;
    i32x8 kf[3];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(krow + 256 * DH + 128 * i + 32 * g16);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(krow + 256 * DH + 128 * i + 32 * g16 + 16);
      kf[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    if (ROPE && DH == 0) {
      const unsigned char* kr = krow + G::ROPE_OFF + 32 * (g16 & 1);   // inside the row
      const u32x4 lo = *reinterpret_cast<const u32x4*>(kr);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(kr + 16);
      const bool live = g16 < 2;
      kf[2] = i32x8{live ? (int)lo[0] : 0, live ? (int)lo[1] : 0, live ? (int)lo[2] : 0,
                    live ? (int)lo[3] : 0, live ? (int)hi[0] : 0, live ? (int)hi[1] : 0,
                    live ? (int)hi[2] : 0, live ? (int)hi[3] : 0};
    }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      f32x4 t = mfma_fp8(kf[0], qb[ht][0], f32x4{0.f, 0.f, 0.f, 0.f});
      t = mfma_fp8(kf[1], qb[ht][1], t);
      if (ROPE && DH == 0) t = mfma_fp8(kf[2], qb[ht][2], t);
      sk[ht] = t;
    }
    return;
  } else {
  f32x4 t0[2], t1[2], tr[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    t0[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    t1[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    tr[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (FMT == kFmtBf16) {
    // bf16 K fragments (16 bytes per lane) straight into bf16 MFMA; no scales.
    const unsigned char* krow = raw + (kt * 16 + c16) * RS + 2 * (256 * DH + 8 * g16);
    bf16x8 kf[8];
#pragma unroll
    for (int i = 0; i < kQkAhead; ++i) kf[i] = *reinterpret_cast<const bf16x8*>(krow + 64 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + kQkAhead < 8)
        kf[i + kQkAhead] = *reinterpret_cast<const bf16x8*>(krow + 64 * (i + kQkAhead));
      if (i < 4) {
        t0[0] = mfma_bf16(kf[i], qb[0][i], t0[0]);
        t0[1] = mfma_bf16(kf[i], qb[1][i], t0[1]);
      } else {
        t1[0] = mfma_bf16(kf[i], qb[0][i], t1[0]);
        t1[1] = mfma_bf16(kf[i], qb[1][i], t1[1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ROPE) {
      const bf16x8 kr = *reinterpret_cast<const bf16x8*>(
          raw + (kt * 16 + c16) * RS + G::ROPE_OFF + 2 * (32 * DH + 8 * g16));
      const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(qr_lane);
      const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(qr_lane + 16 * kQRS);
      tr[0] = mfma_bf16(kr, q0, tr[0]);
      tr[1] = mfma_bf16(kr, q1, tr[1]);
    }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) sk[ht] = (t0[ht] + t1[ht]) + tr[ht];
    return;
  }
  static_assert(FMT == kFmtBf16, "fp8_ds_mla tiles take qk_tile_fp8");
  }
}

// Both key sub-tiles of an fp8_ds_mla tile, partial S^T written to this wave's exchange
// slot.  LDS reads are issued while earlier matrix work runs, into registers that consumed
// K words free: the RoPE fragments after the fourth latent k-step; the scales after the
// fourth (NoPE) or after the last (RoPE: no registers earlier); the next sub-tile's K words
// as soon as this one's are consumed (NoPE only, for the same reason).  Each placement
// measured faster than reading at use (C3: RoPE -2.5 %, NoPE -4.7 %), with no spills.
template <int ROPE, int DH>
__device__ __forceinline__ void qk_tile_fp8(const unsigned char* raw, const __bf16* qr_lane,
                                            const bf16x8 (&qb)[2][8], f32x4* mine, int lane,
                                            int g16, int c16) {
  constexpr int RS = MlaGeom<ROPE, kFmtFp8>::RS;
  constexpr int ROPE_OFF = MlaGeom<ROPE, kFmtFp8>::ROPE_OFF;
  constexpr int kRopeAt = 4, kScaleAt = ROPE ? 8 : 4;   // k-step before which they are read
  constexpr bool kNextEarly = ROPE == 0;
  u32x4 kw[4];
  auto load_k = [&](int kt) {
    const unsigned char* krow = raw + (2 * c16 + kt) * RS + 256 * DH + 16 * g16;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) kw[jj] = *reinterpret_cast<const u32x4*>(krow + 64 * jj);
  };
  load_k(0);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    f32x4 t0[2], t1[2], tr[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      t0[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      t1[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      tr[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 kr, q0, q1;
    f32x2 sc[4];   // scales of keys 4 g + j of the sub-tile (LDS rows 2 (4 g + j) + kt)
    auto load_rope = [&]() {
      kr = *reinterpret_cast<const bf16x8*>(raw + (2 * c16 + kt) * RS + ROPE_OFF +
                                            2 * (32 * DH + 8 * g16));
      q0 = *reinterpret_cast<const bf16x8*>(qr_lane);
      q1 = *reinterpret_cast<const bf16x8*>(qr_lane + 16 * kQRS);
    };
    auto load_sc = [&]() {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sc[j] = *reinterpret_cast<const f32x2*>(raw + (2 * (4 * g16 + j) + kt) * RS +
                                                kScaleOff + 8 * DH);
    };
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (ROPE && i == kRopeAt) load_rope();
      if (i == kScaleAt) load_sc();
      const u32x4 w = kw[i >> 1];
      const bf16x4 lo = e4m3x4_to_bf16((i & 1) ? w[2] : w[0]);
      const bf16x4 hi = e4m3x4_to_bf16((i & 1) ? w[3] : w[1]);
      const bf16x8 k{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (i < 4) {
        t0[0] = mfma_bf16(k, qb[0][i], t0[0]);
        t0[1] = mfma_bf16(k, qb[1][i], t0[1]);
      } else {
        t1[0] = mfma_bf16(k, qb[0][i], t1[0]);
        t1[1] = mfma_bf16(k, qb[1][i], t1[1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kNextEarly && kt == 0) load_k(1);
    if (kScaleAt >= 8) load_sc();
    if (ROPE) {
      tr[0] = mfma_bf16(kr, q0, tr[0]);
      tr[1] = mfma_bf16(kr, q1, tr[1]);
    }
    f32x4 sk[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sk[ht][j] = fmaf(t1[ht][j], sc[j][1], fmaf(t0[ht][j], sc[j][0], tr[ht][j]));
    mine[(2 * kt) * kWave + lane] = sk[0];
    mine[(2 * kt + 1) * kWave + lane] = sk[1];
    if (!kNextEarly && kt == 0) load_k(1);
  }
}

// O^T[256 DH .. +255][32 heads] += V^T P^T for the bf16 rows.
template <int ROPE, int FMT, int DH>
__device__ __forceinline__ void pv_part(const unsigned char* raw, const float (&pv)[2][2][4],
                                        f32x4 (&o_acc)[2][16], bool& sc_bad, int g16,
                                        int c16) {
  constexpr int RS = MlaGeom<ROPE, FMT>::RS;
  if constexpr (FMT == kFmtBf16) {
    // V^T from the bf16 rows by ds_read_b64_tr_b16: lane (g, i) supplies keys {4g + i/4}
    // (then 16 + ...) x dims {16 dt + 4 (i%4) .. +3}, receives dim 16 dt + i of keys
    // 4g .. 4g+3 (lo) and 16 + 4g .. (hi); decoded to fp16 for the fp16 MFMA.
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const unsigned char* vbase =
        raw + (4 * g16 + (c16 >> 2)) * RS + 2 * (256 * DH + 4 * (c16 & 3));
    f16x8 pb[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[ht][e] = (_Float16)pv[ht][e >> 2][e & 3];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      __builtin_amdgcn_sched_barrier(0);
      const unsigned char* src = vbase + 32 * dt;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(const_cast<unsigned char*>(src)));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(const_cast<unsigned char*>(src + 16 * RS)));
      const f16x8 va = bf16x8_to_f16(lo, hi);
      o_acc[0][dt] = mfma_f16(va, pb[0], o_acc[0][dt]);
      o_acc[1][dt] = mfma_f16(va, pb[1], o_acc[1][dt]);
    }
    __builtin_amdgcn_sched_barrier(0);
    (void)sc_bad;
    return;
  }
  static_assert(FMT == kFmtBf16, "e4m3-coded rows take pv_tile");
}

// PV of the e4m3-coded rows (fp8_ds_mla and plain E4M3) over the wave's two 128-dim blocks
// as one stream of 16 fragment steps: the transposed V reads run four steps ahead across the
// block boundary, and the second block's scales (fp8_ds_mla) are read while the first
// block's matrix work runs.  Plain E4M3 rows have no per-key scales: P as is, the
// per-tensor scale applied to the normalised output.  V^T fragments come straight from the
// e4m3 rows through ds_read_b64_tr_b8: in lane group g, lane pair (2e, 2e+1) addresses the
// LDS row of P^T's K-index e (bytes 8 (lane & 1) of the fragment's 16 dims), and lane (g, i)
// receives dim i of those eight rows -- the key order of the P^T operand taken from the S^T
// accumulators in place.  V's per-128 scale is folded into P per block.
template <int ROPE, int FMT, int DH>
__device__ __forceinline__ void pv_tile(const unsigned char* raw, const float (&pv)[2][2][4],
                                        f32x4 (&o_acc)[2][16], bool& sc_bad, int g16, int c16) {
  static_assert(FMT == kFmtFp8 || FMT == kFmtE4m3, "e4m3-coded rows");
  constexpr int RS = MlaGeom<ROPE, FMT>::RS;
  constexpr bool SC = FMT == kFmtFp8;
  // LDS row of P^T's K-index e in lane group g: key 4 g + (e & 3) of sub-tile e >> 2
  // (fp8_ds_mla tiles interleave the two sub-tiles' rows).
  auto kp_row = [&](int e) {
    return SC ? 2 * (4 * g16 + (e & 3)) + (e >> 2) : 16 * (e >> 2) + 4 * g16 + (e & 3);
  };
  const unsigned char* vbase = raw + kp_row(c16 >> 1) * RS + 256 * DH + 8 * (c16 & 1);
  typedef int v2i __attribute__((ext_vector_type(2)));
  auto read_v = [&](int d) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(const_cast<unsigned char*>(vbase + 16 * d)));
  };
  float vsc[8];
  auto load_sc = [&](int b2) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vsc[e] = *reinterpret_cast<const float*>(raw + kp_row(e) * RS + kScaleOff +
                                               4 * (2 * DH + b2));
  };
  f16x8 pb[2];
  auto make_pb = [&]() {
    if constexpr (SC) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sc_bad |= !(fabsf(vsc[e]) <= kMaxVScale);
    }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[ht][e] = SC ? (_Float16)(pv[ht][e >> 2][e & 3] * vsc[e])
                       : (_Float16)pv[ht][e >> 2][e & 3];
  };
  v2i vw[4];
  if (SC) load_sc(0);
#pragma unroll
  for (int d = 0; d < 4; ++d) vw[d] = read_v(d);
  make_pb();
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    __builtin_amdgcn_sched_barrier(0);
    if (SC && d == 8) make_pb();
    const v2i w = vw[d & 3];
    if (d + 4 < 16) vw[d & 3] = read_v(d + 4);
    if (SC && d == 4) load_sc(1);
    const f16x4 lo = e4m3x4_to_f16((uint32_t)w[0]), hi = e4m3x4_to_f16((uint32_t)w[1]);
    const f16x8 va{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    o_acc[0][d] = mfma_f16(va, pb[0], o_acc[0][d]);
    o_acc[1][d] = mfma_f16(va, pb[1], o_acc[1][d]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int ROPE, int FMT, bool TG>
__global__ __launch_bounds__(kMlaThreads) void k_mla_fp8(MlaLaunch a, int nsplit,
                                                         int keys_per_split, float* part) {
  using G = MlaGeom<ROPE, FMT, TG>;
  static_assert(!TG || FMT != kFmtBf16, "two wave groups take the e4m3-coded rows");
  constexpr int NT = kMlaThreads;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f32x4* xs = reinterpret_cast<f32x4*>(smem + G::OFF_XS);
  __bf16* qr_sh = reinterpret_cast<__bf16*>(smem + G::OFF_QR);
  int* slot_sh = reinterpret_cast<int*>(smem + G::OFF_SLOT);
  uint32_t* mask_sh = reinterpret_cast<uint32_t*>(smem + G::OFF_MASK);
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;

  const int tid = threadIdx.x, tid0 = tid;
  const int lane0 = tid & (kWave - 1);
  const int wave = tid >> 6;
  // Partners (same heads, other latent half) are waves 2 pair and 2 pair + 1.  One group:
  // head group hg = pair; with fewer than 128 heads the idle head groups are the high ones,
  // so the active waves spread over the four SIMDs (wave w runs on SIMD w % 4).  Two groups
  // (TG, at most 64 heads): waves 4 grp .. 4 grp + 3, head group hg = pair & 1.
  const int pair = wave >> 1, dh = wave & 1;
  const int grp = TG ? wave >> 2 : 0;
  const int hg = TG ? pair & 1 : pair;
  const int r = blockIdx.x;
  constexpr int HPW = TG ? 64 : kHeadsPerWg;   // heads per work-group
  const int hbase = blockIdx.y * HPW;
  const int h0 = hbase + hg * 32;
  const int split = blockIdx.z;
  const SeqView& s = a.s;
  const int H = a.n_heads;
  // This split's top-k indices, up to kMaxSplitKeys / NT per thread (entry i = tid + NT u),
  // are loaded first, clamped to the row's top_k entries, so that they are in flight with
  // the request lookup below; the row's length masks them afterwards.
  constexpr int SPT = kMaxSplitKeys / NT;
  const int k_begin = split * keys_per_split;
  const int32_t* sel = a.window > 0 ? nullptr : a.idx + (size_t)r * a.top_k;
  int tv[SPT];
  if (sel) {
#pragma unroll
    for (int u = 0; u < SPT; ++u) tv[u] = sel[min(k_begin + tid + NT * u, a.top_k - 1)];
  }
  const int b = request_of_wave(s.q_start, s.batch, r);
  const int p = s.q_pos[r];
  bool row_ok = true;
  if (p < 0 || p >= s.seq_lens[b] || p >= s.max_seq_len) {
    if (tid == 0 && blockIdx.y == 0 && split == 0) raise_fault(a.fault, kFaultQpos);
    row_ok = false;
  }
  // Selected keys: the row's top-k list, or in window mode the last `window` positions.
  int nsel = a.window > 0 ? min(a.window, p + 1) : a.len[r];
  if (nsel < 0 || nsel > a.top_k) {
    if (tid == 0 && blockIdx.y == 0 && split == 0) raise_fault(a.fault, kFaultTopk);
    nsel = max(0, min(nsel, a.top_k));
  }
  if (!row_ok) nsel = 0;
  const int k_end = min(nsel, k_begin + keys_per_split);
  const int nkeys = max(0, k_end - k_begin);
  const int ntiles = (nkeys + kTK - 1) / kTK;

  // Physical slot of every selected key of this split (-1: outside [0, p] or bad block).
  // Every block-table entry is loaded in one round (block 0 for a position outside [0, p],
  // masked afterwards) rather than one dependent round per entry.
  const int32_t* bt = s.block_table + (size_t)b * s.mbps;
  const int nent = ntiles * kTK;
  bool bad_t = false, bad_b = false;
  if (nkeys > 0) {
    const unsigned long long num_blocks = (unsigned long long)a.num_blocks;
    const int wbase = p - nsel + 1 + k_begin;
    int bv[SPT];
    if (!sel) {
#pragma unroll
      for (int u = 0; u < SPT; ++u) tv[u] = wbase + tid + NT * u;
    }
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const bool t_ok = tv[u] >= 0 && tv[u] <= p;
      bv[u] = bt[t_ok ? tv[u] >> s.lbs : 0];
    }
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int i = tid + NT * u;
      const int t = tv[u];
      int slot = -1;
      if (i < nkeys) {
        if (t < 0 || t > p) bad_t = true;
        else if ((unsigned long long)(unsigned)bv[u] >= num_blocks) bad_b = true;
        else slot = (bv[u] << s.lbs) | (t & ((1 << s.lbs) - 1));
      }
      if (i < nent) slot_sh[i] = slot;
      // Bit k of a tile's mask: its k-th selected key has a slot.  A wave's 64 entries are
      // two whole tiles (i - lane is a multiple of 64), so one ballot gives both masks.
      const uint64_t ok = __ballot(slot >= 0);
      if (lane0 == 0 && i < nent) {
        mask_sh[i >> 5] = (uint32_t)ok;
        if ((i >> 5) + 1 < ntiles) mask_sh[(i >> 5) + 1] = (uint32_t)(ok >> 32);
      }
    }
  }
  if (bad_t) raise_fault(a.fault, kFaultTopk);
  if (bad_b) raise_fault(a.fault, kFaultBlock);
  // RoPE query of the group's heads (bf16, as given) into LDS.
  if (ROPE && FMT != kFmtE4m3) {
    for (int i = tid; i < HPW * 8; i += NT) {
      const int hh = i >> 3, q8 = i & 7;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (hbase + hh < H)
        v = *reinterpret_cast<const u32x4*>(
            static_cast<const __bf16*>(a.q) + ((size_t)r * H + hbase + hh) * 576 + 512 + 8 * q8);
      *reinterpret_cast<u32x4*>(qr_sh + hh * kQRS + 8 * q8) = v;
    }
  }
  __syncthreads();

  // Gather: instruction m of a tile moves chunks 64m .. 64m+63 of the tile's rows into LDS
  // block m (chunk f = key f / NCH, bytes 16 (f % NCH) of its row); lanes past the tile or
  // on a masked key read zeros instead.  Every wave issues exactly PER_WAVE transfers per
  // tile, which the vmcnt waits below rely on.
  const uint8_t* pool = static_cast<const uint8_t*>(a.pool);
  const uint8_t* zero_row = g_zero_row;
  asm volatile("" : "+s"(zero_row));   // loaded once, not re-fetched from the GOT per tile
  auto issue = [&](int tile, int lane) {
    const uint32_t stage = lds0 + (uint32_t)((tile % G::NSTAGE) * G::STAGE);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int slot[G::PER_WAVE], off[G::PER_WAVE];
#pragma unroll
    for (int u = 0; u < G::PER_WAVE; ++u) {
      const int f = (wv + u * kMlaWaves) * kWave + lane;
      const int kk = min(f / G::NCH, kTK - 1);
      off[u] = 16 * (f - (f / G::NCH) * G::NCH);
      slot[u] = slot_sh[tile * kTK + kk];
      if (f >= G::RAW) slot[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < G::PER_WAVE; ++u) {
      const int m = wv + u * kMlaWaves;
      const uint8_t* src =
          slot[u] >= 0 ? pool + (int64_t)slot[u] * G::ROW_BYTES + off[u] : zero_row;
      const uint32_t dst = m < G::NBLK ? stage + (uint32_t)(m * 1024) : lds0 + G::OFF_JUNK;
      dma16(src, dst);
    }
  };

  // Latent query fragments for this wave's 32 heads and dim half (B operand of S^T = K Q^T).
  const int g16 = lane0 >> 4, c16 = lane0 & 15;
  const bool ht_live[2] = {h0 < H, h0 + 16 < H};
  const bool active = ht_live[0];
  typename QFrag<FMT>::type qb[2][QFrag<FMT>::N];
  bool q_range = true;
  float qks[2] = {1.0f, 1.0f};   // logit scale per head (lane column)
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int hq = ht_live[ht] ? h0 + 16 * ht + c16 : c16;
    if constexpr (FMT == kFmtE4m3) {
      // E4M3 codes [r][h][512 + ROPE]; value = code * q_scale[r][h].
      const uint8_t* qh = static_cast<const uint8_t*>(a.q) + ((size_t)r * H + hq) * (512 + ROPE);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        u32x4 lo = u32x4{0, 0, 0, 0}, hi = u32x4{0, 0, 0, 0};
        const bool live = i < 2 || (ROPE && dh == 0 && g16 < 2);
        const uint8_t* src = i < 2 ? qh + 256 * dh + 128 * i + 32 * g16 : qh + 512 + 32 * g16;
        if (live) {
          lo = *reinterpret_cast<const u32x4*>(src);
          hi = *reinterpret_cast<const u32x4*>(src + 16);
        }
        qb[ht][i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      const float qs = a.q_scale[(size_t)r * H + hq];
      q_range &= fabsf(qs) <= 3.4028235e38f;   // finite
      qks[ht] = a.kv_scale * qs;
      continue;
    } else {
    const __bf16* qh = static_cast<const __bf16*>(a.q) + ((size_t)r * H + hq) * (512 + ROPE) +
                       256 * dh;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // k-step i's dims: fp8_ds_mla rows pair k-steps in 16-byte reads (dims 64 (i/2) +
      // 16 g + 8 (i%2) ..), bf16 rows take dims 32 i + 8 g ..
      const int qo = FMT == kFmtFp8 ? 64 * (i >> 1) + 16 * g16 + 8 * (i & 1) : 32 * i + 8 * g16;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qh + qo);
      qb[ht][i] = v;                     // bf16 MFMA, the query as given
      if constexpr (FMT == kFmtFp8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) q_range &= fabsf((float)v[e]) <= 3.4028235e38f;   // finite
      }
    }
    }
  }
  if (__any(!q_range) && active && lane0 == 0) raise_fault(a.fault, kFaultRange);
  const float qk_scale = a.softmax_scale * ssmax_mult(a.ssmax_s, row_ok ? p : 0) * kLog2e;
  qks[0] *= qk_scale;
  qks[1] *= qk_scale;
  if constexpr (FMT != kFmtE4m3) {
    // The scale is zero only under SSMax at position 0, where the row has one key and every
    // positive scale gives the same softmax; the smallest normal float keeps masked keys'
    // -inf logits at -inf (0 * -inf would be NaN).
    qks[0] = fmaxf(qks[0], 1.17549435e-38f);
    qks[1] = fmaxf(qks[1], 1.17549435e-38f);
  }

  f32x4 o_acc[2][16];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int i = 0; i < 16; ++i) o_acc[ht][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
  float l_part[2] = {0.f, 0.f};
  bool sc_bad = false;   // a latent scale that could push P * scale out of fp16

  // One tile's phases.  Lane-derived addresses are recomputed every tile (a few VALU
  // instructions) rather than hoisted out of the loop: the query and the accumulator leave
  // no registers to keep them.
  auto opaque_lane = [&]() {
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    return lane;
  };
  auto tile_raw = [&](int tile) {
    return smem + (tile % G::NSTAGE) * G::STAGE;
  };
  // QK: this wave's partial S^T of the tile into its exchange slot.
  auto do_qk = [&](int tile, f32x4* xsb) {
    const int lane = opaque_lane();
    const int g16 = lane >> 4, c16 = lane & 15;
    const unsigned char* raw = tile_raw(tile);
    // Partial S^T over this wave's dims per key sub-tile, exchanged through LDS; both
    // partner waves then add half 0 + half 1 in the same order.
    {
      const __bf16* qr_lane = qr_sh + (hg * 32 + c16) * kQRS + 32 * dh + 8 * g16;
      f32x4* mine = xsb + wave * 4 * kWave;
      if constexpr (FMT == kFmtFp8) {
        if (dh == 0) qk_tile_fp8<ROPE, 0>(raw, qr_lane, qb, mine, lane, g16, c16);
        else qk_tile_fp8<ROPE, 1>(raw, qr_lane, qb, mine, lane, g16, c16);
      } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 sk[2];
        if (dh == 0) qk_part<ROPE, FMT, 0>(raw, qr_lane, qb, kt, sk, g16, c16);
        else qk_part<ROPE, FMT, 1>(raw, qr_lane, qb, kt, sk, g16, c16);
        mine[(2 * kt) * kWave + lane] = sk[0];
        mine[(2 * kt + 1) * kWave + lane] = sk[1];
      }
      }
    }
  };
  // Softmax and PV of the tile, from both halves' partial S in the exchange buffer.
  auto do_smpv = [&](int tile, const f32x4* xsb) {
    const int lane = opaque_lane();
    const int g16 = lane >> 4, c16 = lane & 15;
    const unsigned char* raw = tile_raw(tile);
    // Both halves' partial S of this wave's heads and the tile's key mask, read after the
    // barrier.  (Reading them before the gather of tile + 2 is issued spills.)
    f32x4 ps0[2][2], ps1[2][2];
    uint32_t vmask = 0;
    auto load_partials = [&]() {
      const f32x4* p0 = xsb + (2 * pair) * 4 * kWave;
      const f32x4* p1 = xsb + (2 * pair + 1) * 4 * kWave;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          ps0[kt][ht] = p0[(2 * kt + ht) * kWave + lane];
          ps1[kt][ht] = p1[(2 * kt + ht) * kWave + lane];
        }
      vmask = mask_sh[tile];
    };
    load_partials();
    // Logits: half 0 + half 1 in the same order in both partners.  With a positive logit
    // scale c (every format but plain E4M3, whose per-head query scale may take any sign) c
    // is applied inside the exponent's fma and the tile maximum is max(s) * c; otherwise the
    // scaled logits are formed first.
    constexpr bool FOLD = FMT != kFmtE4m3;
    float pv[2][2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const f32x4 sum = ps0[kt][ht] + ps1[kt][ht];
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[ht][kt][j] = FOLD ? sum[j] : sum[j] * qks[ht];
      }
    // Keys without a slot (a tile's tail, masked keys) are rare: one uniform test skips the
    // per-key masking for whole tiles.  Accumulator key (kt, 4 g + j) is selection index
    // 8 g + 2 j + kt with the interleaved rows of fp8_ds_mla tiles, 16 kt + 4 g + j otherwise.
    if (__builtin_amdgcn_readfirstlane(vmask) != 0xFFFFFFFFu) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int bit = FMT == kFmtFp8 ? 8 * g16 + 2 * j + kt : 16 * kt + 4 * g16 + j;
          if (!((vmask >> bit) & 1u)) pv[0][kt][j] = pv[1][kt][j] = -__builtin_inff();
        }
    }
    auto weight = [&](int ht, int kt, int j, float msub) {
      return FOLD ? __builtin_amdgcn_exp2f(fmaf(pv[ht][kt][j], qks[ht], -msub))
                  : __builtin_amdgcn_exp2f(pv[ht][kt][j] - msub);
    };

    // ---- online softmax (base 2) per head (lane column), identical in both partner waves.
    //      The vector-only phase runs at wave priority 1 (measured 1.5 % faster per tile than
    //      leaving both waves of a SIMD at one priority; raising the matrix phases instead
    //      gained nothing).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      // The weights are taken against the running maximum before the tile's own maximum is
      // known (the two are independent); only when the tile raises the maximum by more
      // than the slack -- rare after the first tile -- are they taken again.
      const float msub0 = (m_run[ht] == -__builtin_inff()) ? 0.f : m_run[ht];
      float ev[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) ev[kt][j] = weight(ht, kt, j, msub0);
      float mt = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mt = fmaxf(mt, pv[ht][kt][j]);
      mt = max_over_lane_groups(mt);
      // max(s) * c == max(s * c) for c > 0 (rounding is monotonic).
      if (FOLD) mt *= qks[ht];
      const bool need = mt > m_run[ht] + kRescaleSlack || (m_run[ht] == -__builtin_inff() && mt > m_run[ht]);
      if (__any(need)) {
        const float m_new = need ? fmaxf(m_run[ht], mt) : m_run[ht];
        const float alpha = (m_run[ht] == -__builtin_inff()) ? 0.f : exp2f(m_run[ht] - m_new);
        l_part[ht] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[ht][i] *= alpha;
        m_run[ht] = m_new;
        // With no finite logit yet every value is -inf and exp2(-inf - 0) = 0.
        const float msub = (m_new == -__builtin_inff()) ? 0.f : m_new;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) ev[kt][j] = weight(ht, kt, j, msub);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pv[ht][kt][j] = ev[kt][j];
          l_part[ht] += ev[kt][j];
        }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- O^T += V^T P^T over this wave's dim half
    if constexpr (FMT == kFmtBf16) {
      if (dh == 0) pv_part<ROPE, FMT, 0>(raw, pv, o_acc, sc_bad, g16, c16);
      else pv_part<ROPE, FMT, 1>(raw, pv, o_acc, sc_bad, g16, c16);
    } else {
      if (dh == 0) pv_tile<ROPE, FMT, 0>(raw, pv, o_acc, sc_bad, g16, c16);
      else pv_tile<ROPE, FMT, 1>(raw, pv, o_acc, sc_bad, g16, c16);
    }
  };

  if constexpr (TG) {
    // Two wave groups over one set of at most 64 heads: waves 0-3 take the even tiles,
    // waves 4-7 the odd ones, each group with its own softmax state, merged at the end.
    // Per step two tiles: [wait for them, barrier, gather the next two] [QK] [barrier]
    // [softmax, PV].  The ring holds two steps (four tile slots); one exchange buffer,
    // the groups on disjoint wave slots.
    for (int t = 0; t < 2; ++t)
      if (t < ntiles) issue(t, lane0);
    const int nsteps = (ntiles + 1) / 2;
    for (int st = 0; st < nsteps; ++st) {
      const int tile = __builtin_amdgcn_readfirstlane(2 * st + grp);   // wave-uniform
      const bool mine_ok = active && tile < ntiles;
      wait_vmcnt<0>();
      __syncthreads();   // this step's tiles are in LDS; every wave is done with the last
      for (int t = 2 * st + 2; t < 2 * st + 4; ++t)
        if (t < ntiles) issue(t, opaque_lane());
      if (mine_ok) do_qk(tile, xs);
      __syncthreads();   // partial S published
      if (mine_ok) do_smpv(tile, xs);
    }
  } else {
  if constexpr (G::ONEBAR) {
    if (ntiles > 0) issue(0, lane0);
    if (ntiles > 1) issue(1, lane0);
    if (ntiles > 1) wait_vmcnt<G::PER_WAVE>();
    else wait_vmcnt<0>();
    __syncthreads();   // tile 0 is in LDS
  } else {
#pragma unroll
    for (int t = 0; t < G::NSTAGE - 1; ++t)
      if (t < ntiles) issue(t, lane0);
  }
  for (int tile = 0; tile < ntiles; ++tile) {
    if constexpr (!G::ONEBAR) {
      // Two-tile ring: this tile's transfers are the only outstanding ones.
      static_assert(G::NSTAGE == 2, "the wait below assumes one tile in flight");
      wait_vmcnt<0>();
      __syncthreads();   // the tile is in LDS; every wave is done with the previous tile
      if (tile + G::NSTAGE - 1 < ntiles) issue(tile + G::NSTAGE - 1, opaque_lane());
    }
    f32x4* xsb = xs + (G::ONEBAR ? (tile & 1) * G::XS_WORDS : 0);
    // Waves whose heads are all past n_heads only move data and keep the barriers.
    if (active) do_qk(tile, xsb);
    if constexpr (G::ONEBAR) {
      // Only tile + 1's transfers are outstanding.  After the barrier every wave's partial
      // S of this tile and tile + 1 are in LDS, and every wave is done with tile - 1, whose
      // ring slot takes tile + 2.
      wait_vmcnt<0>();
      __syncthreads();
      if (tile + 2 < ntiles) issue(tile + 2, opaque_lane());
    } else {
      __syncthreads();
    }
    if (active) do_smpv(tile, xsb);
  }
  }

  if (__any(sc_bad) && lane0 == 0) raise_fault(a.fault, kFaultRange);

  if constexpr (TG) {
    // Group 1's softmax state (running maximum, partial sums, accumulator) through LDS to
    // its group-0 counterpart (same heads, same dims, same lane layout), which rescales
    // both to the larger maximum and adds them; one head tile at a time.
    constexpr int kItems = 2 + 16 * 4;
    static_assert(4 * kItems * kWave * 4 <= G::BYTES, "merge area");
    float* mg = reinterpret_cast<float*>(smem) + (wave & 3) * kItems * kWave + lane0;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      __syncthreads();   // every wave is done with the ring / the previous head tile
      if (grp == 1 && active) {
        mg[0] = m_run[ht];
        mg[kWave] = l_part[ht];
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) mg[(2 + 4 * i + j) * kWave] = o_acc[ht][i][j];
      }
      __syncthreads();
      if (grp == 0 && active) {
        const float m1 = mg[0], l1 = mg[kWave];
        const float M = fmaxf(m_run[ht], m1);
        const float a0 = m_run[ht] == -__builtin_inff() ? 0.f : exp2f(m_run[ht] - M);
        const float a1 = m1 == -__builtin_inff() ? 0.f : exp2f(m1 - M);
        l_part[ht] = l_part[ht] * a0 + l1 * a1;
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o_acc[ht][i][j] = o_acc[ht][i][j] * a0 + mg[(2 + 4 * i + j) * kWave] * a1;
        m_run[ht] = M;
      }
    }
    if (grp == 1) return;
  }

  // ---- epilogue: lane (g, i) holds O[head h0 + 16 ht + i][dims 256 dh + 16 t + 4 g + j]
  if (!active) return;
  const int g16e = lane0 >> 4, c16e = lane0 & 15;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    if (!ht_live[ht]) continue;
    const float l = sum_over_lane_groups(l_part[ht]);
    const int h = h0 + 16 * ht + c16e;
    // Plain E4M3 rows: V's per-tensor scale multiplies the normalised sum.
    const float inv = l > 0.f ? (FMT == kFmtE4m3 ? a.kv_scale : 1.0f) / l : 0.f;
    const float lse2 = l > 0.f ? m_run[ht] + log2f(l) : -__builtin_inff();
    const int d0 = 256 * dh + 4 * g16e;
    if (nsplit == 1) {
      __bf16* out = static_cast<__bf16*>(a.out) + ((size_t)r * H + h) * 512 + d0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const f32x4 v = o_acc[ht][i] * inv;
        *reinterpret_cast<bf16x4*>(out + 16 * i) =
            bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      }
      if (a.lse && g16e == 0 && dh == 0) a.lse[(size_t)r * H + h] = lse2 * kLn2;
    } else {
      float* po = part + (((size_t)r * H + h) * nsplit + split) * 513;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const f32x4 v = o_acc[ht][i] * inv;
        *reinterpret_cast<f32x4*>(po + d0 + 16 * i) = v;
      }
      if (g16e == 0 && dh == 0) po[512] = lse2;
    }
  }
  (void)tid0;
  (void)g16;
  (void)c16;
}

template <int ROPE, int FMT, bool TG>
constexpr size_t mla_lds_bytes() {
  return (size_t)MlaGeom<ROPE, FMT, TG>::BYTES;
}

// Merge split partials: o = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M) (base-2 lse).
// The partial outputs of the first kMergeAhead splits are loaded before their weights are
// known, together with every split's lse (one memory round trip for the usual split
// counts); the weights are taken one split per lane, their sum and the weighted sum in
// split order.
constexpr int kMaxSplits = (kMaxSplitKeys + kTK - 1) / kTK;
constexpr int kMergeAhead = 16;
static_assert(kMaxSplits <= kWave, "one split per lane of the first wave");
__global__ __launch_bounds__(128) void k_mla_combine(MlaLaunch a, int nsplit, const float* part) {
  __shared__ float wsh[kMaxSplits];
  __shared__ float Msh, Lsh;
  const int r = blockIdx.x, h = blockIdx.y;
  const int H = a.n_heads;
  const float* base = part + ((size_t)r * H + h) * nsplit * 513;
  const int d = 4 * threadIdx.x;
  f32x4 v[kMergeAhead];
#pragma unroll
  for (int u = 0; u < kMergeAhead; ++u) {
    const float* o = base + u * 513 + d;
    v[u] = u < nsplit ? f32x4{o[0], o[1], o[2], o[3]} : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (threadIdx.x < kWave) {
    const int sp = threadIdx.x;
    const float l = sp < nsplit ? base[sp * 513 + 512] : -__builtin_inff();
    const float M = wave_max(l);
    if (sp < nsplit) wsh[sp] = l == -__builtin_inff() ? 0.f : exp2f(l - M);
    if (sp == 0) Msh = M;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float L = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) L += wsh[sp];
    Lsh = L;
  }
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeAhead; ++u)
    if (u < nsplit) acc += wsh[u] * v[u];
  for (int sp0 = kMergeAhead; sp0 < nsplit; sp0 += 4) {
    f32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* o = base + (sp0 + u) * 513 + d;
      w[u] = sp0 + u < nsplit ? f32x4{o[0], o[1], o[2], o[3]} : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (sp0 + u < nsplit) acc += wsh[sp0 + u] * w[u];
  }
  __syncthreads();
  const float M = Msh, L = Lsh;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  acc *= inv;
  __bf16* out = static_cast<__bf16*>(a.out) + ((size_t)r * H + h) * 512 + d;
  *reinterpret_cast<bf16x4*>(out) = bf16x4{(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
  if (a.lse && threadIdx.x == 0)
    a.lse[(size_t)r * H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -__builtin_inff();
}

// fp32 format: [512 latent][64 RoPE] fp32 per token, fp32 queries and outputs.  One
// work-group per (row, head); two-pass softmax over at most 2048 logits held in LDS.
__global__ __launch_bounds__(256) void k_mla_f32(MlaLaunch a) {
  __shared__ float qsh[576];
  __shared__ float logit[2048];
  __shared__ int slot_sh[2048];
  __shared__ float red[8];
  const int r = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const SeqView& s = a.s;
  const int H = a.n_heads;
  const int D = 512 + a.rope_dim;
  const int b = request_of(s.q_start, s.batch, r);
  int p = s.q_pos[r];
  bool row_ok = true;
  if (p < 0 || p >= s.seq_lens[b] || p >= s.max_seq_len) {
    if (tid == 0 && h == 0) raise_fault(a.fault, kFaultQpos);
    row_ok = false;
  }
  int n = a.len[r];
  if (n < 0 || n > a.top_k) {
    if (tid == 0 && h == 0) raise_fault(a.fault, kFaultTopk);
    n = max(0, min(n, a.top_k));
  }
  if (!row_ok) n = 0;
  const float* q = static_cast<const float*>(a.q) + ((size_t)r * H + h) * D;
  for (int i = tid; i < D; i += 256) qsh[i] = q[i];
  const float scale = a.softmax_scale * ssmax_mult(a.ssmax_s, row_ok ? p : 0);
  const int32_t* sel = a.idx + (size_t)r * a.top_k;
  const int32_t* bt = s.block_table + (size_t)b * s.mbps;
  for (int i = tid; i < n; i += 256) {
    const int t = sel[i];
    int slot = -1;
    if (t < 0 || t > p) {
      if (h == 0) raise_fault(a.fault, kFaultTopk);
    } else {
      const int blk = bt[t >> s.lbs];
      if ((unsigned)blk >= (unsigned long long)a.num_blocks) {
        if (h == 0) raise_fault(a.fault, kFaultBlock);
      } else {
        slot = (blk << s.lbs) | (t & ((1 << s.lbs) - 1));
      }
    }
    slot_sh[i] = slot;
  }
  __syncthreads();
  const float* pool = static_cast<const float*>(a.pool);
  float mx = -__builtin_inff();
  for (int i = tid; i < n; i += 256) {
    float v = -__builtin_inff();
    if (slot_sh[i] >= 0) {
      const float* row = pool + (size_t)slot_sh[i] * 576;
      float d = 0.f;
      for (int k = 0; k < 512; ++k) d = fmaf(qsh[k], row[k], d);
      for (int k = 0; k < a.rope_dim; ++k) d = fmaf(qsh[512 + k], row[512 + k], d);
      v = d * scale;
    }
    logit[i] = v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int i = tid; i < n; i += 256) {
    const float e = (logit[i] == -__builtin_inff()) ? 0.f : expf(logit[i] - mx);
    logit[i] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = sum;
  __syncthreads();
  sum = red[4] + red[5] + red[6] + red[7];
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  float* out = static_cast<float*>(a.out) + ((size_t)r * H + h) * 512;
  for (int d = tid; d < 512; d += 256) {
    float acc = 0.f;
    for (int i = 0; i < n; ++i)
      if (slot_sh[i] >= 0) acc = fmaf(logit[i], pool[(size_t)slot_sh[i] * 576 + d], acc);
    out[d] = acc * inv;
  }
  if (a.lse && tid == 0)
    a.lse[(size_t)r * H + h] = sum > 0.f ? mx + logf(sum) : -__builtin_inff();
}

struct MlaPlan {
  int groups, nsplit, keys_per_split;
};

// One work-group per (row, 128 heads, key split); splits only when the grid would leave
// CUs idle.
MlaPlan plan_mla(const SeqView& s, int H, int top_k, bool tg) {
  MlaPlan pl{};
  const int hpw = tg ? 64 : kHeadsPerWg;
  pl.groups = (H + hpw - 1) / hpw;
  const long long base = (long long)s.total_q * pl.groups;
  // >= 4 tiles per split: below that the partials (2 KB per row, head and split, written
  // and read back) and each split's copy of the row's queries outweigh the extra CUs
  // (8 decode rows: 56 -> 44 us against 2-tile splits).
  const int max_split = max(1, (top_k + 4 * kTK - 1) / (4 * kTK));
  int ns = 1;
  while (ns < max_split && base * ns < 256) ns <<= 1;
  ns = min(ns, max_split);
  pl.nsplit = ns;
  const int per = (top_k + ns - 1) / ns;
  pl.keys_per_split = (per + kTK - 1) / kTK * kTK;
  return pl;
}

// The two-wave-group form (64 heads per work-group) serves at most 64 heads, and more heads
// whenever 128-head work-groups would leave CUs idle (few decode rows): each row then takes
// twice the work-groups, with every wave busy (8 decode rows at 32k: 41.9 -> 37.6 us; one
// row at 1M positions: 35.5 -> 29.7 us).  Rows of bf16 cache lines keep one group.
bool use_two_groups(const SeqView& s, int H, int top_k, bool bf16_rows) {
  if (bf16_rows) return false;
  if (H <= 64) return true;
  const MlaPlan one = plan_mla(s, H, top_k, false);
  return (long long)s.total_q * one.groups * one.nsplit < 256;
}

template <int ROPE, int FMT, bool TG>
hipError_t launch_rows_tg(const MlaLaunch& a, const MlaPlan& pl, float* part, hipStream_t st) {
  constexpr size_t lds = mla_lds_bytes<ROPE, FMT, TG>();
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mla_fp8<ROPE, FMT, TG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid(a.s.total_q, pl.groups, pl.nsplit);
  k_mla_fp8<ROPE, FMT, TG><<<grid, kMlaThreads, lds, st>>>(a, pl.nsplit, pl.keys_per_split,
                                                           part);
  return hipGetLastError();
}

// At most 64 heads use half the waves of a 128-head work-group; two wave groups then take
// alternate tiles of the row (measured at 64 / 16 heads on the 64k verify selections:
// 171.8 -> 135.0 us / 150.8 -> 118.5 us).
template <int ROPE, int FMT>
hipError_t launch_rows(const MlaLaunch& a, bool tg, const MlaPlan& pl, float* part,
                       hipStream_t st) {
  if constexpr (FMT != kFmtBf16) {
    if (tg) return launch_rows_tg<ROPE, FMT, true>(a, pl, part, st);
  }
  return launch_rows_tg<ROPE, FMT, false>(a, pl, part, st);
}

}  // namespace

// Enough for either work-group form (the row format is not an argument here).
size_t mla_ws_bytes(const SeqView& s, int n_heads, int top_k) {
  const int ns = max(plan_mla(s, n_heads, top_k, false).nsplit,
                     plan_mla(s, n_heads, top_k, true).nsplit);
  if (ns <= 1) return 0;
  return align_up((size_t)s.total_q * n_heads * ns * 513 * sizeof(float), 256);
}

hipError_t launch_mla(const MlaLaunch& a, hipStream_t st) {
  if (!a.fp8) {
    k_mla_f32<<<dim3(a.s.total_q, a.n_heads), 256, 0, st>>>(a);
    return hipGetLastError();
  }
  const bool tg = use_two_groups(a.s, a.n_heads, a.top_k, a.bf16_rows);
  const MlaPlan pl = plan_mla(a.s, a.n_heads, a.top_k, tg);
  float* part = pl.nsplit > 1 ? static_cast<float*>(a.ws) : nullptr;
  hipError_t e;
  if (a.bf16_rows)
    e = a.rope_dim ? launch_rows<64, kFmtBf16>(a, false, pl, part, st)
                   : launch_rows<0, kFmtBf16>(a, false, pl, part, st);
  else if (a.e4m3_rows)
    e = a.rope_dim ? launch_rows<64, kFmtE4m3>(a, tg, pl, part, st)
                   : launch_rows<0, kFmtE4m3>(a, tg, pl, part, st);
  else
    e = a.rope_dim ? launch_rows<64, kFmtFp8>(a, tg, pl, part, st)
                   : launch_rows<0, kFmtFp8>(a, tg, pl, part, st);
  if (e != hipSuccess || pl.nsplit <= 1) return e;
  k_mla_combine<<<dim3(a.s.total_q, a.n_heads), 128, 0, st>>>(a, pl.nsplit, part);
  return hipGetLastError();
}

}  // namespace ml4
