// Decode: one new query per sequence against a KV cache, optionally split over the cache
// ("split-K") with a merge pass.
//
// Method: the KV-cache decode step of ninaddeshpande.com "Transformer internals: attention
// without the mysticism" ("The KV cache and the memory wall"): each query row attends to every
// cached key; the cache holds already-rotated keys and is used as stored, the query is rotated
// (devthesis.com section 3) at its own position.  The G = Hq/Hkv query heads that share a KV head
// (codingpancake.com section 6.1) are processed together so each K/V byte is read once.
//
// decode_split_kernel, one workgroup per (sequence, KV head, group of up to 16 query heads, split):
//  * The G query heads of a KV head fill the 16 columns of the MFMA B operand.  More than 16
//    (multi-query attention) go to decode_wide_kernel (decode_wide.hip), which shares each K/V
//    tile among up to 64 of them; only a cache or pool over 2 GiB, beyond that kernel's 32-bit
//    offsets, comes here with G > 16: the query heads are then taken 16 at a time by separate
//    workgroups on consecutive slots of one XCD (workgroup ids are dealt to the 8 XCDs in turn),
//    so their reads of the same K/V meet in that XCD's L2.
//  * The waves stream disjoint 32-key sub-blocks of the split; loads of sub-block i+1 are in
//    flight while sub-block i is consumed (16 x 16-byte loads per lane).  The cache is read once,
//    so its loads are nontemporal (streaming) and do not displace reusable lines in the caches.
//  * Scores S^T = K q^T on v_mfma_f32_16x16x32_bf16: K goes from HBM straight into the A
//    operand; the G query rows (padded to 16) form the B operand.  The rotated, scaled query is
//    split into bf16 hi + lo parts and multiplied twice, so q keeps ~16 significant bits and K is
//    used exactly.  The matrix cores are nearly idle in this memory-bound pass.
//  * Online softmax per row in log2 units (row max over the 4 lane groups with permlane swaps),
//    lazy rescaling as in prefill.
//  * O^T += V^T P^T on the same MFMA shape; V^T comes from a wave-private LDS tile through
//    ds_read_b64_tr_b16.
//  * The waves' (m, l, O) are merged through LDS.  With one split (8 waves per workgroup, used
//    when there are enough (sequence, KV head) pairs to fill the GPU) the workgroup writes o and
//    lse directly; otherwise (4 waves per workgroup) it writes one partial per (row, split).
// decode_merge_kernel, one workgroup per (sequence, query head), only after a split cache:
// combines the splits with the same log-sum-exp algebra and writes o and lse.
//
// Paged cache (PAGED): the cache is a pool of fixed-size blocks [num_blocks, Hkv, bs, D] found
// through a per-sequence block table (codingpancake.com "Building Self-Attention and Transformer
// Engines", section 6.2).  bs is a power of two >= 16, so each 16-key half of a wave's 32-key
// sub-block lies in one block: the two block ids are wave-uniform scalars, fetched one sub-block
// ahead of the loads that use them, and every lane's K/V address is the block's base plus its
// slot, exactly as in the contiguous cache.
//
// Sliding window (codingpancake.com section 6.4): only cache rows j >= q_pos[b] - window are
// visible.  Each split starts at the first 32-key sub-block holding a visible row; the rows
// before the window in that sub-block are masked, and their values are never used (zeroed), so
// blocks before the window may already have been released and reused.
#include "common.h"

namespace attn {

namespace {

constexpr int kWavesSplit = 4;   // waves per workgroup when the cache is split (merge pass after)
constexpr int kWavesWhole = 8;   // waves per workgroup when one workgroup covers the whole cache
constexpr int kSub = 32;   // keys per wave iteration
constexpr int kNumXcd = 8;  // workgroup ids are dealt to the XCDs in turn
constexpr float kRescaleThreshold = 8.0f;

// max / sum partners across the 16-lane rows of a wave.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int vswz(int r, int lc) {  // 16 chunks per row (D = 128)
  return lc ^ (((r & 3) << 2) | ((r >> 2) & 3));
}

// NW waves per workgroup.  WHOLE: one split covers the whole cache, and the workgroup writes the
// final o (OUT_BF16 selects its type) and lse itself; otherwise it writes one partial (m, l, O)
// per (row, split) for decode_merge_kernel.
// STREAM: one workgroup per (sequence, KV head, split), and K/V read once (nontemporal loads);
// off when several workgroups share a KV head (more than 16 query heads per KV head): their ids
// are then placed on one XCD and their repeated reads should stay in L2.  WIN: sliding window.
template <int D, bool ROPE, int NW, bool WHOLE, bool OUT_BF16, bool PAGED, bool STREAM, bool WIN>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ cache_len, const int32_t* __restrict__ q_pos, int B, int Hq, int Hkv,
    int S_max, const float2* __restrict__ table, int table_max_pos, int n_split, int chunk,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, void* __restrict__ o, float* __restrict__ lse,
    const int32_t* __restrict__ block_table, int max_blocks, int bs_log2, int num_blocks, int window) {
  constexpr int kWaves = NW;
  constexpr int kThreads = NW * 64;
  constexpr int NCH = D / 8;
  constexpr int KS = D / 32;        // MFMA k-steps over D
  constexpr int DB = D / 16;        // 16-wide output blocks over D
  constexpr int LPT = kSub * NCH / 64;  // 16-byte loads of K (and of V) per lane per sub-block
  static_assert(D == 128 || D == 64, "head dim");

  // Per-wave V tile; after the key loop each wave reuses its own tile (same bytes) to publish
  // its O^T for the cross-wave merge: 16 rows x D floats == 32 keys x D bf16.
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kWaves][kSub * D];
  __shared__ float red_ml[kWaves][16][2];

  const int G = Hq / Hkv;
  int split, hkv, b, sub;
  if constexpr (STREAM) {
    // grid (n_split, Hkv, B): one group of query heads per KV head
    split = blockIdx.x;
    hkv = blockIdx.y;
    b = blockIdx.z;
    sub = 0;
  } else {
    // workgroup id -> (unit, sub-group): the n_sub workgroups of a unit share id % 8 (one XCD)
    const int n_sub = (G + 15) / 16;             // groups of 16 query heads per KV head
    const int n_units = n_split * Hkv * B;
    const int wid = blockIdx.x;
    const int jx = wid / kNumXcd;
    sub = jx % n_sub;
    const int unit = (jx / n_sub) * kNumXcd + wid % kNumXcd;
    if (unit >= n_units) return;
    split = unit % n_split;
    hkv = (unit / n_split) % Hkv;
    b = unit / (n_split * Hkv);
  }
  const int h0 = hkv * G + sub * 16;             // first query head of this workgroup
  const int Gs = min(16, G - sub * 16);          // query heads of this workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int qrow = i16;  // this lane's query row in the group (B-operand column / C column)

  int L = cache_len[b];
  L = L < 0 ? 0 : (L > S_max ? S_max : L);
  // first visible row (sliding window); q_pos is given whenever a window is
  const int wstart = WIN ? max(q_pos[b] - window, 0) : 0;
  const int kbeg = max(split * chunk, wstart & ~(kSub - 1));
  const int kend0 = min(split * chunk + chunk, L);
  // nothing visible in this split: empty range (then every sub-block processed below holds at
  // least one visible row, the first one holding wstart)
  const int kend = wstart < kend0 ? kend0 : 0;
  // checked build, site 0: the workgroup's (sequence, KV head, split, query heads) and key range
  if (!ATTN_IN(b < B && hkv < Hkv && split < n_split && h0 >= 0 && h0 + max(Gs, 1) <= Hq && kbeg >= 0 &&
                   kend <= S_max,
               0))
    return;

  // ---- query fragments (hi/lo bf16), rotated at q_pos[b] and scaled by log2(e)/sqrt(D) ----
  bf16x8 qhi[KS], qlo[KS];
  {
    const float qscale = 1.4426950408889634f / sqrtf((float)D);
    int pos = 0;
    if constexpr (ROPE) {
      pos = q_pos[b];
      if (pos < 0 || pos >= table_max_pos) pos = 0;  // such rows are written as NaN at the end
    }
    const bool valid = qrow < Gs;
    const uint16_t* qp = q + ((int64_t)b * Hq + h0 + (valid ? qrow : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 32 * ks + 8 * g16;
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + d0);
      if (!valid) w = u32x4{0, 0, 0, 0};
      float x[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) { x[2 * t] = bf16lo(w[t]); x[2 * t + 1] = bf16hi(w[t]); }
      if constexpr (ROPE) {
        const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)pos * (D / 2) + d0 / 2);
        const f32x4 c01 = tp[0], c23 = tp[1];
        const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float c = cs[2 * p], s = cs[2 * p + 1];
          const float x0 = x[2 * p], x1 = x[2 * p + 1];
          x[2 * p] = x0 * c - x1 * s;
          x[2 * p + 1] = x0 * s + x1 * c;
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float xs = x[t] * qscale;
        const __bf16 hi = (__bf16)xs;
        qhi[ks][t] = hi;
        qlo[ks][t] = (__bf16)(xs - (float)hi);
      }
    }
  }

  // contiguous: rows of this (sequence, KV head); paged: the block pool (rows found per block)
  const int64_t kv_off = PAGED ? 0 : ((int64_t)b * Hkv + hkv) * S_max * D;
  const uint16_t* kg = kc + kv_off;
  const uint16_t* vg = vc + kv_off;
  const int32_t* btr = block_table + (PAGED ? (int64_t)b * max_blocks : 0);
  const int bmask = (1 << bs_log2) - 1;
  // Paged: pool row of the first key of each 16-key half of the sub-block at k0 (a half past the
  // end of the cache reuses the first half's block, so every address stays inside a block).
  auto half_rows = [&](int k0, int64_t& r0, int64_t& r1) {
    const int k0u = wave_uniform(k0);
    // checked build, site 2: the block table entries read lie in this sequence's row of the table
    int blk0 = wave_uniform(btr[ATTN_IN((k0u >> bs_log2) < max_blocks, 2) ? k0u >> bs_log2 : 0]);
    int blk1 = blk0;
    const int k1 = k0u + 16;
    if (k1 < kend) blk1 = wave_uniform(btr[ATTN_IN((k1 >> bs_log2) < max_blocks, 2) ? k1 >> bs_log2 : 0]);
    blk0 = min(max(blk0, 0), num_blocks - 1);
    blk1 = min(max(blk1, 0), num_blocks - 1);
    r0 = (((int64_t)blk0 * Hkv + hkv) << bs_log2) + (k0u & bmask);
    r1 = k1 < kend ? (((int64_t)blk1 * Hkv + hkv) << bs_log2) + (k1 & bmask) : r0;
  };

  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // K: lane loads key (kb*16 + i16), 16 B at d = 32 ks + 8 g16  -> A operand directly.
  // V: lane loads chunk c = lane + 64 i of the 32 x D tile (row c / NCH, chunk c % NCH).
  u32x4 kst[2][KS], vst[LPT];
  // r0, r1: paged only (pool rows of the two halves); the contiguous cache ignores them.
  auto issue = [&](int k0, int64_t r0, int64_t r1) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = k0 + kb * 16 + i16;
      const bool ok = key < kend && key >= wstart;
      int64_t row;
      if constexpr (PAGED) row = ok ? (kb ? r1 : r0) + i16 : r0;
      else row = ok ? key : kbeg;
      // checked build, site 1: the key row inside the cache (or the pool)
      row = ATTN_IN(row >= 0 && row < (PAGED ? ((int64_t)num_blocks * Hkv << bs_log2) : (int64_t)S_max), 1) ? row : 0;
      const uint16_t* kp = kg + row * D + 8 * g16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4* src = reinterpret_cast<const u32x4*>(kp + 32 * ks);
        kst[kb][ks] = STREAM ? __builtin_nontemporal_load(src) : *src;
      }
    }
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = lane + 64 * i;
      const int key = k0 + c / NCH;
      const bool ok = key < kend && key >= wstart;
      int64_t row;
      if constexpr (PAGED) row = ok ? ((c / NCH) >= 16 ? r1 : r0) + ((c / NCH) & 15) : r0;
      else row = ok ? key : kbeg;
      // checked build, site 1: the value row inside the cache (or the pool)
      row = ATTN_IN(row >= 0 && row < (PAGED ? ((int64_t)num_blocks * Hkv << bs_log2) : (int64_t)S_max), 1) ? row : 0;
      const u32x4* src = reinterpret_cast<const u32x4*>(vg + row * D + (c % NCH) * 8);
      vst[i] = STREAM ? __builtin_nontemporal_load(src) : *src;
      if (!ok) vst[i] = u32x4{0, 0, 0, 0};
    }
  };

  ATTN_LDS uint16_t* vl = (ATTN_LDS uint16_t*)(v_lds[wave]);
  const int nsub = kend > kbeg ? (kend - kbeg + kSub - 1) / kSub : 0;
  int it = wave;
  int64_t nr0 = 0, nr1 = 0;  // paged: pool rows of the next sub-block to issue
  if constexpr (PAGED) {
    if (it < nsub) half_rows(kbeg + it * kSub, nr0, nr1);
  }
  if (it < nsub) issue(kbeg + it * kSub, nr0, nr1);
  if constexpr (PAGED) {
    if (it + kWaves < nsub) half_rows(kbeg + (it + kWaves) * kSub, nr0, nr1);
  }
  for (; it < nsub; it += kWaves) {
    const int k0 = kbeg + it * kSub;
    // consume staged registers
    u32x4 kcur[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kcur[kb][ks] = kst[kb][ks];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = lane + 64 * i;
      const int r = c / NCH, cc = c % NCH;
      const int off = r * D + (D == 128 ? vswz(r, cc) : (cc ^ (r & 7))) * 8;
      *reinterpret_cast<ATTN_LDS u32x4*>(vl + off) = vst[i];
    }
    if (it + kWaves < nsub) {
      issue(k0 + kWaves * kSub, nr0, nr1);
      // the block ids of the sub-block after that are fetched now, a whole iteration ahead
      if constexpr (PAGED) {
        if (it + 2 * kWaves < nsub) half_rows(k0 + 2 * kWaves * kSub, nr0, nr1);
      }
    }

    // scores
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, kcur[kb][ks]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[ks], sacc[kb], 0, 0, 0);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[ks], sacc[kb], 0, 0, 0);
      }
    }
    if (k0 + kSub > kend || k0 < wstart) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + kb * 16 + 4 * g16 + r;
          if (key >= kend || key < wstart) sacc[kb][r] = -INFINITY;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleThreshold) != 0) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    bf16x8 pf;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float p = fast_exp2(sacc[t >> 2][t & 3] - m_run);
      l_run += p;
      pf[t] = (__bf16)p;
    }
    // O^T += V^T P^T ; key order inside the contraction: t -> (t/4)*16 + 4*g16 + t%4
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 a;
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        const int vr = tg * 16 + 4 * g16 + (i16 >> 2);
        const int lc = 2 * db + ((i16 & 3) >> 1);
        const int off = vr * D + (D == 128 ? vswz(vr, lc) : (lc ^ (vr & 7))) * 8 + 4 * (i16 & 1);
        const i16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<ATTN_LDS i16x4*>(vl + off));
        const bf16x4 wb = __builtin_bit_cast(bf16x4, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * tg + e] = wb[e];
      }
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[db], 0, 0, 0);
    }
  }

  // ---- combine the 4 waves ----
  l_run = sum_xor32(sum_xor16(l_run));
  if (lane < 16) {
    red_ml[wave][qrow][0] = m_run;
    red_ml[wave][qrow][1] = l_run;
  }
  ATTN_LDS float* red_o = (ATTN_LDS float*)(&v_lds[0][0]);  // [wave][16][D]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[(wave * 16 + qrow) * D + db * 16 + 4 * g16 + r] = oacc[db][r];
  __syncthreads();

  // thread -> (row, d) pairs of the merged partial
  for (int e = tid; e < Gs * D; e += kThreads) {
    const int rr = e / D, d = e % D;
    if (!ATTN_IN(h0 + rr < Hq, 3)) continue;  // checked build, site 3: the output row
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_ml[w][rr][0]);
    float Lsum = 0.f, acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = fast_exp2(red_ml[w][rr][0] - M);
        Lsum += red_ml[w][rr][1] * sc;
        acc += red_o[(w * 16 + rr) * D + d] * sc;
      }
    }
    if constexpr (WHOLE) {
      float out = Lsum > 0.f ? acc / Lsum : 0.f;
      float ls = Lsum > 0.f ? (M + log2f(Lsum)) * 0.6931471805599453f : -INFINITY;
      if constexpr (ROPE) {
        const int p = q_pos[b];
        if (p < 0 || p >= table_max_pos) { out = __builtin_nanf(""); ls = __builtin_nanf(""); }
      }
      const int64_t oi = ((int64_t)b * Hq + h0 + rr) * D + d;
      if constexpr (OUT_BF16) {
        reinterpret_cast<__bf16*>(o)[oi] = (__bf16)out;
      } else {
        reinterpret_cast<float*>(o)[oi] = out;
      }
      if (lse && d == 0) lse[(int64_t)b * Hq + h0 + rr] = ls;
    } else {
      const int64_t part = (((int64_t)b * Hq + h0 + rr) * n_split + split);
      ws_o[part * D + d] = acc;
      if (d == 0) {
        ws_ml[part * 2 + 0] = M;
        ws_ml[part * 2 + 1] = Lsum;
      }
    }
  }
}

template <int D, bool OUT_BF16, bool ROPE>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, const int32_t* __restrict__ q_pos,
    int table_max_pos, int Hq, int n_split, void* __restrict__ o, float* __restrict__ lse) {
  constexpr int kGroup = 8;  // partials whose loads are in flight together
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  if (!ATTN_IN(h < Hq && d < D, 4)) return;  // checked build, site 4: the merged row
  const int64_t base = ((int64_t)b * Hq + h) * n_split;
  // One pass over the splits, kGroup at a time, rescaling the running sum to each group's max.
  float M = -INFINITY, Lsum = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += kGroup) {
    float m[kGroup], l[kGroup], x[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const bool in = s0 + i < n_split;
      const int64_t part = base + (in ? s0 + i : 0);
      m[i] = in ? ws_ml[part * 2] : -INFINITY;
      l[i] = ws_ml[part * 2 + 1];
      x[i] = ws_o[part * D + d];
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) Mg = fmaxf(Mg, m[i]);
    if (Mg == -INFINITY) continue;  // nothing seen yet (empty splits)
    const float r = fast_exp2(M - Mg);  // 0 while M is -inf
    Lsum *= r;
    acc *= r;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float sc = fast_exp2(m[i] - Mg);  // 0 for empty splits and those past n_split
      Lsum += l[i] * sc;
      acc += x[i] * sc;
    }
    M = Mg;
  }
  float out = Lsum > 0.f ? acc / Lsum : 0.f;
  float ls = Lsum > 0.f ? (M + log2f(Lsum)) * 0.6931471805599453f : -INFINITY;
  if constexpr (ROPE) {
    const int p = q_pos[b];
    if (p < 0 || p >= table_max_pos) { out = __builtin_nanf(""); ls = __builtin_nanf(""); }
  }
  const int64_t oi = ((int64_t)b * Hq + h) * D + d;
  if constexpr (OUT_BF16) {
    reinterpret_cast<__bf16*>(o)[oi] = (__bf16)out;
  } else {
    reinterpret_cast<float*>(o)[oi] = out;
  }
  if (lse && d == 0) lse[(int64_t)b * Hq + h] = ls;
}

template <int D, bool ROPE, bool PAGED, bool STREAM, bool WIN>
hipError_t go(const DecodeArgs& a, hipStream_t st) {
  const uint16_t* q = (const uint16_t*)a.q;
  const uint16_t* kc = (const uint16_t*)a.k;
  const uint16_t* vc = (const uint16_t*)a.v;
  const float2* tab = reinterpret_cast<const float2*>(a.table);
  const int n_sub = (a.Hq / a.Hkv + 15) / 16;
  const int64_t n_units = (int64_t)a.n_split * a.Hkv * a.B;
  const dim3 grid = STREAM ? dim3(a.n_split, a.Hkv, a.B)
                           : dim3((unsigned)(((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * n_sub));
  if (a.n_split == 1) {
    // one workgroup per (sequence, KV head, query group) streams the whole cache and writes o itself
    if (a.out_bf16)
      hipLaunchKernelGGL((decode_split_kernel<D, ROPE, kWavesWhole, true, true, PAGED, STREAM, WIN>), grid,
                         dim3(64 * kWavesWhole), 0, st, q, kc, vc, a.cache_len, a.q_pos, a.B, a.Hq, a.Hkv, a.S_max,
                         tab, a.table_max_pos, 1, a.chunk, a.ws_o, a.ws_ml, a.o, a.lse, a.block_table,
                         a.max_blocks, a.bs_log2, a.num_blocks, a.window);
    else
      hipLaunchKernelGGL((decode_split_kernel<D, ROPE, kWavesWhole, true, false, PAGED, STREAM, WIN>), grid,
                         dim3(64 * kWavesWhole), 0, st, q, kc, vc, a.cache_len, a.q_pos, a.B, a.Hq, a.Hkv, a.S_max,
                         tab, a.table_max_pos, 1, a.chunk, a.ws_o, a.ws_ml, a.o, a.lse, a.block_table,
                         a.max_blocks, a.bs_log2, a.num_blocks, a.window);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_split_kernel<D, ROPE, kWavesSplit, false, false, PAGED, STREAM, WIN>),
                     grid, dim3(64 * kWavesSplit), 0, st, q, kc, vc, a.cache_len, a.q_pos,
                     a.B, a.Hq, a.Hkv, a.S_max, tab, a.table_max_pos, a.n_split, a.chunk, a.ws_o, a.ws_ml, a.o, a.lse,
                     a.block_table, a.max_blocks, a.bs_log2, a.num_blocks, a.window);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_merge(a, st);
}

template <bool PAGED, bool STREAM, bool WIN>
hipError_t go_d(const DecodeArgs& a, hipStream_t st) {
  const bool rope = a.table != nullptr;
  if (a.D == 64) return rope ? go<64, true, PAGED, STREAM, WIN>(a, st) : go<64, false, PAGED, STREAM, WIN>(a, st);
  return rope ? go<128, true, PAGED, STREAM, WIN>(a, st) : go<128, false, PAGED, STREAM, WIN>(a, st);
}

template <bool PAGED>
hipError_t go_w(const DecodeArgs& a, hipStream_t st) {
  const bool stream = a.Hq / a.Hkv <= 16;
  if (a.window < kNoWindow) return stream ? go_d<PAGED, true, true>(a, st) : go_d<PAGED, false, true>(a, st);
  return stream ? go_d<PAGED, true, false>(a, st) : go_d<PAGED, false, false>(a, st);
}

}  // namespace

ATTN_CHECK_READER(checked_word_decode)

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  // more than 16 query heads per KV head: the shared-tile kernel (its byte offsets are 32-bit)
  if (decode_wide_fits(a)) return launch_decode_wide(a, st);
  return a.block_table ? go_w<true>(a, st) : go_w<false>(a, st);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t st) {
  const bool rope = a.table != nullptr;
  auto go_m = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(a.Hq, a.B), dim3(a.D), 0, st, a.ws_o, a.ws_ml, a.q_pos, a.table_max_pos, a.Hq,
                       a.n_split, a.o, a.lse);
    return hipGetLastError();
  };
  if (a.D == 64) {
    if (a.out_bf16) return rope ? go_m(decode_merge_kernel<64, true, true>) : go_m(decode_merge_kernel<64, true, false>);
    return rope ? go_m(decode_merge_kernel<64, false, true>) : go_m(decode_merge_kernel<64, false, false>);
  }
  if (a.out_bf16) return rope ? go_m(decode_merge_kernel<128, true, true>) : go_m(decode_merge_kernel<128, true, false>);
  return rope ? go_m(decode_merge_kernel<128, false, true>) : go_m(decode_merge_kernel<128, false, false>);
}

}  // namespace attn
