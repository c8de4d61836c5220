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
// One work-group = one query row x a group of heads x a contiguous range of its selected
// keys.  Per 32-key tile:
//   gather  the selected 656-byte rows (slot = block_table[t / bs] * bs + t % bs) with 16-byte
//           loads, decode the e4m3 codes exactly to bf16 and store [key][576] in LDS, keeping
//           the four per-128 scales in fp32 beside them (the RoPE part is already bf16; a
//           NoPE layer never touches those bytes);
//   QK      S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 with keys on M and heads on N, the query
//           fragments resident in registers; each 128-column block is accumulated on its
//           own and multiplied by its key's scale in fp32;
//   softmax online, base 2, per head = per lane column; the running maximum is only moved
//           when a tile exceeds it by more than 2^8, so the accumulator is rarely rescaled;
//   PV      O^T = V^T . P^T on v_mfma_f32_16x16x32_f16 with latent columns on M, heads on
//           N: the V^T fragments come from a second [key][512] fp16 copy of the tile through
//           ds_read_b64_tr_b16, P^T comes from the QK accumulators in place (the key order of
//           both operands is the same permutation), and the per-128 scale of V is folded into
//           P per column block.  fp16 rather than bf16 for this product: e4m3 values are exact
//           in both, and P keeps 11 significant bits instead of 8, which bounds the output
//           error by 2^-11 * sum_t p_t |c_t| even when SSMax makes the softmax peaked.
// A row's selected keys may be split across work-groups; the partial results are merged by
// their log-sum-exp in a second kernel.
#include "ml4_device.h"

namespace ml4 {

namespace {

constexpr int kLatRow = 656;
constexpr int kTK = 32;            // keys per tile
constexpr int kKS = 584;           // bf16 stride of a key row of the QK tile (576 + 8)
constexpr int kVS = 520;           // fp16 stride of a key row of the PV tile (512 + 8)
constexpr float kRescaleSlack = 8.0f;
constexpr uint32_t kFaultBlock = 1u << 0;
constexpr uint32_t kFaultTopk = 1u << 1;
constexpr uint32_t kFaultQpos = 1u << 3;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) short lds_short;

struct Gathered {
  u32x4 lat[4];   // 64 e4m3 codes
  u32x4 rope;     // 8 bf16
  float scale;
  int ok;
};

constexpr int kMlaWaves = 4;
constexpr int kMlaHT = 1;                 // 16-head tiles per wave
constexpr int kHeadsPerWg = kMlaWaves * 16 * kMlaHT;

template <int ROPE, int WAVES, int HT>
__global__ __launch_bounds__(WAVES * kWave) void k_mla_fp8(MlaLaunch a, int nsplit,
                                                           int keys_per_split, float* part) {
  constexpr int NT = WAVES * kWave;
  constexpr int NC = (512 + ROPE) / 32;        // 32-wide K chunks of the QK product
  __shared__ __attribute__((aligned(16))) __bf16 ks_tile[kTK * kKS];
  __shared__ __attribute__((aligned(16))) _Float16 vs_tile[kTK * kVS];
  __shared__ float sc_tile[kTK * 4];
  __shared__ int ok_tile[kTK];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int g16 = lane >> 4, c16 = lane & 15;
  const int r = blockIdx.x;
  const int h0 = blockIdx.y * (WAVES * 16 * HT) + wave * 16 * HT;
  const int split = blockIdx.z;
  const SeqView& s = a.s;
  const int H = a.n_heads;
  const int b = request_of(s.q_start, s.batch, r);
  int p = s.q_pos[r];
  bool row_ok = true;
  if (p < 0 || p >= s.seq_lens[b] || p >= s.max_seq_len) {
    if (tid == 0 && blockIdx.y == 0 && split == 0) raise_fault(a.fault, kFaultQpos);
    row_ok = false;
  }
  int nsel = a.len[r];
  if (nsel < 0 || nsel > a.top_k) {
    if (tid == 0 && blockIdx.y == 0 && split == 0) raise_fault(a.fault, kFaultTopk);
    nsel = max(0, min(nsel, a.top_k));
  }
  if (!row_ok) nsel = 0;
  const int k_begin = split * keys_per_split;
  const int k_end = min(nsel, k_begin + keys_per_split);
  const int ntiles = k_end > k_begin ? (k_end - k_begin + kTK - 1) / kTK : 0;

  // Waves whose heads lie past n_heads only gather.  (n_heads is a multiple of 16.)
  const bool active = h0 < H;
  // Query fragments: B operand of S^T = K Q^T (column = head, K = latent/RoPE dims).
  bf16x8 qb[HT][NC];
  const __bf16* q = static_cast<const __bf16*>(a.q);
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int hq = active ? h0 + ht * 16 + c16 : c16;
    const __bf16* qh = q + ((size_t)r * H + hq) * (512 + ROPE) + 8 * g16;
#pragma unroll
    for (int c = 0; c < NC; ++c) qb[ht][c] = *reinterpret_cast<const bf16x8*>(qh + 32 * c);
  }
  const float qk_scale =
      a.softmax_scale * ssmax_mult(a.ssmax_s, row_ok ? p : 0) * kLog2e;

  f32x4 o_acc[HT][32];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) o_acc[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[HT], l_part[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) { m_run[ht] = -__builtin_inff(); l_part[ht] = 0.f; }

  const int32_t* sel = a.idx + (size_t)r * a.top_k;
  const int32_t* bt = s.block_table + (size_t)b * s.mbps;
  const uint8_t* pool = static_cast<const uint8_t*>(a.pool);
  const int bs_mask = (1 << s.lbs) - 1;

  // Each thread gathers 64 latent codes (+8 RoPE values, +1 scale) of one key per item.
  constexpr int kItems = (kTK * 8 + NT - 1) / NT;
  Gathered gq[kItems];
  auto gather = [&](int tile) {
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int u = tid + it * NT;
      Gathered& G = gq[it];
      G.ok = 0;
      G.scale = 0.f;
      if (u >= kTK * 8) continue;
      const int kk = u >> 3, part = u & 7;
      const int i = k_begin + tile * kTK + kk;
      if (i >= k_end) continue;
      const int t = sel[i];
      if (t < 0 || t > p) {
        if (part == 0) raise_fault(a.fault, kFaultTopk);
        continue;
      }
      const int blk = bt[t >> s.lbs];
      if ((unsigned)blk >= (unsigned long long)a.num_blocks) {
        if (part == 0) raise_fault(a.fault, kFaultBlock);
        continue;
      }
      const uint8_t* rp = pool + (((int64_t)blk << s.lbs) + (t & bs_mask)) * kLatRow;
#pragma unroll
      for (int v = 0; v < 4; ++v) G.lat[v] = *reinterpret_cast<const u32x4*>(rp + 64 * part + 16 * v);
      if (ROPE) G.rope = *reinterpret_cast<const u32x4*>(rp + 528 + 16 * part);
      if (part < 4) G.scale = *reinterpret_cast<const float*>(rp + 512 + 4 * part);
      G.ok = 1;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int u = tid + it * NT;
      if (u >= kTK * 8) continue;
      const Gathered& G = gq[it];
      const int kk = u >> 3, part = u & 7;
      __bf16* dst = ks_tile + kk * kKS + 64 * part;
      _Float16* vdst = vs_tile + kk * kVS + 64 * part;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 x;
          f16x8 y;
          if (G.ok) {
            const bf16x4 lo = e4m3x4_to_bf16(G.lat[v][2 * h]);
            const bf16x4 hi = e4m3x4_to_bf16(G.lat[v][2 * h + 1]);
            x = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const f16x4 flo = e4m3x4_to_f16(G.lat[v][2 * h]);
            const f16x4 fhi = e4m3x4_to_f16(G.lat[v][2 * h + 1]);
            y = f16x8{flo[0], flo[1], flo[2], flo[3], fhi[0], fhi[1], fhi[2], fhi[3]};
          } else {
            x = bf16x8{};
            y = f16x8{};
          }
          *reinterpret_cast<bf16x8*>(dst + 16 * v + 8 * h) = x;
          *reinterpret_cast<f16x8*>(vdst + 16 * v + 8 * h) = y;
        }
      }
      if (ROPE) {
        u32x4 rv = G.ok ? G.rope : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(ks_tile + kk * kKS + 512 + 8 * part) = rv;
      }
      if (part < 4) sc_tile[kk * 4 + part] = G.ok ? G.scale : 0.f;
      if (part == 0) ok_tile[kk] = G.ok;
    }
  };

  if (ntiles > 0) gather(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();   // the previous tile's readers are done
    stage();
    __syncthreads();
    if (tile + 1 < ntiles) gather(tile + 1);   // in flight during this tile's math
    if (!active) continue;

    // ---- S^T = K Q^T : two 16-key sub-tiles x HT 16-head tiles
    f32x4 sacc[2][HT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const __bf16* krow = ks_tile + (kt * 16 + c16) * kKS + 8 * g16;
      float kscale[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) kscale[j][bl] = sc_tile[(kt * 16 + 4 * g16 + j) * 4 + bl];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) sacc[kt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bl = 0; bl < 4; ++bl) {
        f32x4 tmp[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) tmp[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 32 * (4 * bl + c));
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) tmp[ht] = mfma_bf16(ka, qb[ht][4 * bl + c], tmp[ht]);
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int j = 0; j < 4; ++j) sacc[kt][ht][j] = fmaf(tmp[ht][j], kscale[j][bl], sacc[kt][ht][j]);
      }
      if (ROPE) {
#pragma unroll
        for (int c = 16; c < NC; ++c) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 32 * c);
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) sacc[kt][ht] = mfma_bf16(ka, qb[ht][c], sacc[kt][ht]);
        }
      }
    }

    // ---- online softmax (base 2) per head; lane column = head, rows = keys 4*g16 + j
    bool okk[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) okk[kt][j] = ok_tile[kt * 16 + 4 * g16 + j] != 0;
    float pv[2][HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float mt = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = okk[kt][j] ? sacc[kt][ht][j] * qk_scale : -__builtin_inff();
          pv[kt][ht][j] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const bool need = mt > m_run[ht] + kRescaleSlack || (m_run[ht] == -__builtin_inff() && mt > m_run[ht]);
      if (__any(need)) {
        const float m_new = need ? fmaxf(m_run[ht], mt) : m_run[ht];
        const float alpha = (m_run[ht] == -__builtin_inff()) ? 0.f : exp2f(m_run[ht] - m_new);
        l_part[ht] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) o_acc[ht][dt] *= alpha;
        m_run[ht] = m_new;
      }
      const float m_use = m_run[ht];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = (m_use == -__builtin_inff()) ? 0.f : exp2f(pv[kt][ht][j] - m_use);
          pv[kt][ht][j] = e;
          l_part[ht] += e;
        }
    }

    // ---- O^T += V^T P^T, per 128-column block of V with its scale folded into P
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
      f16x8 pb[HT];
      float vs[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) vs[kt][j] = sc_tile[(kt * 16 + 4 * g16 + j) * 4 + bl];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[ht][e] = (_Float16)(pv[e >> 2][ht][e & 3] * vs[e >> 2][e & 3]);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int dt = bl * 8 + dd;
        // lane (g, i) supplies keys {4g + i/4} x dims {16 dt + 4 (i%4) .. +3}; receives dim
        // 16 dt + i of keys 4g .. 4g+3 (then 16 + 4g .. 16 + 4g + 3).
        const _Float16* src0 = vs_tile + (4 * g16 + (c16 >> 2)) * kVS + 16 * dt + 4 * (c16 & 3);
        const _Float16* src1 = src0 + 16 * kVS;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(lds_short*)(const_cast<_Float16*>(src0)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(lds_short*)(const_cast<_Float16*>(src1)));
        const s16x8 w8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const f16x8 va = __builtin_bit_cast(f16x8, w8);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) o_acc[ht][dt] = mfma_f16(va, pb[ht], o_acc[ht][dt]);
      }
    }
  }

  // ---- epilogue: lane (g, i) holds O[head h0 + 16 ht + i][dims 16 dt + 4 g + j]
  if (!active) return;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    float l = l_part[ht];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int h = h0 + ht * 16 + c16;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const float lse2 = l > 0.f ? m_run[ht] + log2f(l) : -__builtin_inff();
    if (nsplit == 1) {
      __bf16* out = static_cast<__bf16*>(a.out) + ((size_t)r * H + h) * 512 + 4 * g16;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const f32x4 v = o_acc[ht][dt] * inv;
        *reinterpret_cast<bf16x4*>(out + 16 * dt) =
            bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      }
      if (a.lse && g16 == 0) a.lse[(size_t)r * H + h] = lse2 * kLn2;
    } else {
      float* po = part + (((size_t)r * H + h) * nsplit + split) * 513;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const f32x4 v = o_acc[ht][dt] * inv;
#pragma unroll
        for (int j = 0; j < 4; ++j) po[16 * dt + 4 * g16 + j] = v[j];
      }
      if (g16 == 0) po[512] = lse2;
    }
  }
}

// Merge split partials: o = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M) (base-2 lse).
__global__ __launch_bounds__(128) void k_mla_combine(MlaLaunch a, int nsplit, const float* part) {
  const int r = blockIdx.x, h = blockIdx.y;
  const int H = a.n_heads;
  const float* base = part + ((size_t)r * H + h) * nsplit * 513;
  float M = -__builtin_inff();
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, base[sp * 513 + 512]);
  float L = 0.f;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  const int d = 4 * threadIdx.x;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float ls = base[sp * 513 + 512];
    if (ls == -__builtin_inff()) continue;
    const float wgt = exp2f(ls - M);
    L += wgt;
    const float* o = base + sp * 513 + d;
    acc += wgt * f32x4{o[0], o[1], o[2], o[3]};
  }
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

MlaPlan plan_mla(const SeqView& s, int H, int top_k) {
  MlaPlan pl{};
  pl.groups = (H + kHeadsPerWg - 1) / kHeadsPerWg;
  const long long base = (long long)s.total_q * pl.groups;
  const int max_split = max(1, (top_k + 2 * kTK - 1) / (2 * kTK));   // >= 2 tiles per split
  int ns = 1;
  while (ns < max_split && base * ns < 256) ns <<= 1;
  ns = min(ns, max_split);
  pl.nsplit = ns;
  const int per = (top_k + ns - 1) / ns;
  pl.keys_per_split = (per + kTK - 1) / kTK * kTK;
  return pl;
}

template <int ROPE>
hipError_t launch_fp8(const MlaLaunch& a, const MlaPlan& pl, float* part, hipStream_t st) {
  dim3 grid(a.s.total_q, pl.groups, pl.nsplit);
  k_mla_fp8<ROPE, kMlaWaves, kMlaHT><<<grid, kMlaWaves * kWave, 0, st>>>(a, pl.nsplit,
                                                                        pl.keys_per_split, part);
  return hipGetLastError();
}

}  // namespace

size_t mla_ws_bytes(const SeqView& s, int n_heads, int top_k) {
  const MlaPlan pl = plan_mla(s, n_heads, top_k);
  if (pl.nsplit <= 1) return 0;
  return align_up((size_t)s.total_q * n_heads * pl.nsplit * 513 * sizeof(float), 256);
}

hipError_t launch_mla(const MlaLaunch& a, hipStream_t st) {
  if (!a.fp8) {
    k_mla_f32<<<dim3(a.s.total_q, a.n_heads), 256, 0, st>>>(a);
    return hipGetLastError();
  }
  const MlaPlan pl = plan_mla(a.s, a.n_heads, a.top_k);
  float* part = pl.nsplit > 1 ? static_cast<float*>(a.ws) : nullptr;
  hipError_t e = a.rope_dim ? launch_fp8<64>(a, pl, part, st) : launch_fp8<0>(a, pl, part, st);
  if (e != hipSuccess || pl.nsplit <= 1) return e;
  k_mla_combine<<<dim3(a.s.total_q, a.n_heads), 128, 0, st>>>(a, pl.nsplit, part);
  return hipGetLastError();
}

}  // namespace ml4
