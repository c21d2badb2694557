// Decode for wide query groups: more than 16 query heads per KV head (multi-query attention has
// one KV head for all of them).
//
// Method: the KV-cache decode step of ninaddeshpande.com "Transformer internals: attention
// without the mysticism" ("The KV cache and the memory wall"), with the query heads of a KV
// head sharing its K/V (codingpancake.com "Building Self-Attention and Transformer Engines",
// section 6.1; devthesis.com "Transformer Architecture & Self-Attention Mechanics", the MQA
// variant), and the sliding window of codingpancake.com section 6.4.
//
// decode_wide_kernel, one workgroup per (sequence, KV head, split, super-group of up to HG x 16
// query heads), NW = 2 * HG waves:
//  * Wave w owns the 16 query heads of head group w % HG (the 16 columns of the MFMA B operand)
//    and the 32-key half w / HG of every 64-key tile.
//  * The K and V tiles go HBM -> LDS once per workgroup (buffer_load_dwordx4 ... lds, no register
//    staging), into kStages stages with kStages - 1 tiles in flight, and all HG head groups read
//    their MFMA operands from there: every K/V byte leaves HBM once for up to HG x 16 query
//    heads.  (The decode kernel for G <= 16 instead loads K straight into registers, one query
//    group per KV head.)
//  * Scores S^T = K q^T on v_mfma_f32_16x16x32_bf16 with the query split into bf16 hi + lo parts
//    (K used exactly), online softmax in log2 units with lazy rescaling, O^T += V^T P^T with V^T
//    read through ds_read_b64_tr_b16: the same arithmetic as the narrow decode kernel.
//  * Rows outside [window start, cache length) inside a tile are loaded from the nearest visible
//    row (finite data) and masked, so rows before the window are never read.
//  * Paged cache (PAGED): the pool [num_blocks, Hkv, bs, D] and the per-sequence block table of
//    codingpancake.com section 6.2.  A 64-key tile spans at most four blocks (bs >= 16); their ids
//    are scalar loads made one tile ahead, and each lane picks the one holding its row.
//  * The two key halves of a head group merge through LDS; the workgroup then writes o and lse
//    (one split) or one partial per (row, split) for the merge pass.
#include "common.h"

namespace attn {

namespace {

constexpr int kTileKeys = 64;   // keys per LDS tile (two 32-key halves)
// LDS stages; kStages - 1 tiles are in flight.  Four (128 KiB, one workgroup per CU) measured
// best: three are as fast, five slower; two stages with two workgroups per CU, slower.
constexpr int kStages = 4;
constexpr int kNumXcd = 8;      // workgroup ids are dealt to the XCDs in turn
constexpr float kRescaleThreshold = 8.0f;
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3: 32-bit data format, raw
// Added to the byte offset of a load past the last tile: beyond any resource range (the ranges are
// under 2^31 - 256 bytes, so the sum neither wraps nor lands inside), so the load moves no data.
constexpr uint32_t kDeadOffset = 0x80000000u;
constexpr int64_t kMaxWideBytes = ((int64_t)1 << 31) - 256;
// Cache policy of the tile loads: the nontemporal bit (each K/V byte is read once).  Measured
// against the default policy: the same at 16 tiles per workgroup, 5.6 -> 6.5 TB/s at 64.
constexpr int kLoadAux = 2;

// s_waitcnt with only vmcnt limited (expcnt 7, lgkmcnt 15): vmcnt sits in bits 3:0 and 15:14.
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

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

// Physical 16-byte chunk of logical chunk lc in LDS row r (an involution in lc): 16 consecutive
// rows read at one logical chunk hit 16 different bank groups.
template <int D>
__device__ __forceinline__ int swz(int r, int lc) {
  if constexpr (D == 128) {
    return lc ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    return lc ^ (r & 7);
  }
}

// Workgroup barrier for the LDS stages.  A fence would make the compiler wait for every
// HBM->LDS load in flight (they write LDS), which would drain the loads of the later tiles; each
// wave instead waits for its own loads of the tile about to be read (vmcnt) before the barrier.
// The asm also keeps the compiler from moving memory accesses across it; lgkmcnt(0) completes
// this wave's LDS reads and writes first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, bool ROPE, int HG, bool WHOLE, bool OUT_BF16, bool PAGED, bool WIN>
__global__ __launch_bounds__(2 * HG * 64) void decode_wide_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ cache_len, const int32_t* __restrict__ q_pos, int B, int Hq, int Hkv,
    int S_max, const float2* __restrict__ table, int table_max_pos, int n_split, int chunk,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, void* __restrict__ o, float* __restrict__ lse,
    const int32_t* __restrict__ block_table, int max_blocks, int bs_log2, int num_blocks, int window) {
  constexpr int NW = 2 * HG;
  constexpr int NCH = D / 8;                    // 16-byte chunks per row
  constexpr int KS = D / 32;                    // MFMA k-steps over D
  constexpr int DB = D / 16;                    // 16-wide output blocks over D
  constexpr int TILE = kTileKeys * D;           // elements per tensor per tile
  constexpr int LPW = TILE * 2 / 1024 / NW;     // 1 KiB wave-loads per tensor per tile
  constexpr int LPT = 2 * LPW;                  // ... for K and V
  constexpr int P = kStages - 1;                // tiles in flight ahead of the one consumed
  static_assert(LPW * 1024 * NW == TILE * 2, "tile split over waves");
  static_assert(D == 128 || D == 64, "head dim");

  // One LDS object per stage and tensor, so that with the stage fixed at compile time the
  // compiler sees that loads into the other stages never alias the operands being read.
  __shared__ __attribute__((aligned(16))) uint16_t st0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t st1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t st2[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t st3[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sv2[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sv3[TILE];
  static_assert(kStages == 4, "four stage objects per tensor");
  static_assert(2 * 16 * D * 4 <= TILE * 2, "two head groups' partial O fit in one K stage");

  // ---- workgroup -> (unit, super-group); the super-groups of a unit share an XCD ----
  const int G = Hq / Hkv;
  const int n_sub = (G + 15) / 16;
  const int n_super = (n_sub + HG - 1) / HG;
  const int n_units = n_split * Hkv * B;
  const int wid = blockIdx.x;
  const int jx = wid / kNumXcd;
  const int sg = jx % n_super;
  const int unit = (jx / n_super) * kNumXcd + wid % kNumXcd;
  if (unit >= n_units) return;
  const int split = unit % n_split;
  const int hkv = (unit / n_split) % Hkv;
  const int b = unit / (n_split * Hkv);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int hg = wave % HG;       // head group of this wave
  const int kw = wave / HG;       // 32-key half of each tile
  const int g16 = lane >> 4, i16 = lane & 15;
  const int sub = sg * HG + hg;
  const int h0 = hkv * G + sub * 16;          // first query head of this wave
  const int Gs = min(16, G - sub * 16);       // its query heads (<= 0: a padding wave)

  int L = cache_len[b];
  L = L < 0 ? 0 : (L > S_max ? S_max : L);
  const int wstart = WIN ? max(q_pos[b] - window, 0) : 0;
  const int kbeg = max(split * chunk, wstart & ~(kTileKeys - 1));
  const int kend0 = min(split * chunk + chunk, L);
  const int kend = wstart < kend0 ? kend0 : 0;   // nothing visible in this split: empty
  const int nt = kend > kbeg ? (kend - kbeg + kTileKeys - 1) / kTileKeys : 0;
  // checked build, site 0: the workgroup's (sequence, KV head, split, super-group) and key range
  if (!ATTN_IN(b < B && hkv < Hkv && split < n_split && sg < n_super && kbeg >= 0 && kend <= S_max, 0)) return;

  // ---- HBM -> LDS: wave-load i of this wave fills chunks [(i * NW + wave) * 64, +64) of the
  // tile; lane L's chunk C holds logical chunk swz(r, C % NCH) of tile row r = C / NCH, read from
  // the nearest visible cache row.  The loads go through buffer resources over this (sequence,
  // KV head)'s rows.  Every step issues one tile's loads, also past the last tile: those get an
  // offset beyond the resource's range, so they move no data and only keep the count of loads
  // in flight the same on every path (each wait below is then a fixed vmcnt). ----
  // contiguous: this (sequence, KV head)'s rows; paged: the whole pool
  const int64_t kv_off = PAGED ? 0 : ((int64_t)b * Hkv + hkv) * S_max * D;
  const uint32_t kv_bytes = PAGED ? (uint32_t)num_blocks * Hkv * (D << bs_log2) * 2 : (uint32_t)S_max * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + kv_off), (short)0, kv_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + kv_off), (short)0, kv_bytes, kBufferWord3);
  int dma_row[LPW], dma_elem[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int C = (i * NW + wave) * 64 + lane;
    dma_row[i] = C / NCH;
    dma_elem[i] = swz<D>(C / NCH, C % NCH) * 8;
  }
  // Paged: ids of the (up to four) blocks holding the visible rows of tile t, as wave-uniform
  // scalar loads (their indices are clamped into the table row; the ids are clamped into the
  // pool only where they are used, so the four loads are in flight together).
  const int32_t* btr = block_table + (PAGED ? (int64_t)b * max_blocks : 0);
  const int jmax = max(kend - 1, 0) >> bs_log2;
  auto tile_blocks = [&](int t, int (&ids)[4]) {
    if constexpr (PAGED) {
      const int k0c = max(min(max(kbeg + t * kTileKeys, wstart), kend - 1), 0);
      const int j0 = wave_uniform(k0c >> bs_log2);
#pragma unroll
      for (int i = 0; i < 4; ++i)  // (clamped where used; checked build, site 2: inside the table row)
        ids[i] = btr[ATTN_IN(min(j0 + i, jmax) < max_blocks, 2) ? min(j0 + i, jmax) : 0];
    }
  };
  auto issue = [&](int t, uint16_t* stage, uint16_t* vstage, const int (&ids)[4]) {
    const int k0 = kbeg + t * kTileKeys;
    // 0 for a tile to load, kDeadOffset past the last tile (an add, not a branch, so that every
    // path issues the same loads)
    const uint32_t dead = (t < nt) ? 0u : kDeadOffset;
    const int j0 = max(min(max(k0, wstart), kend - 1), 0) >> bs_log2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int key = max(min(max(k0 + dma_row[i], wstart), kend - 1), 0);
      uint32_t row;
      if constexpr (PAGED) {
        const int jj = (key >> bs_log2) - j0;  // 0 .. 3
        int blk = jj == 0 ? ids[0] : jj == 1 ? ids[1] : jj == 2 ? ids[2] : ids[3];
        blk = min(max(blk, 0), num_blocks - 1);
        row = ((uint32_t)(blk * Hkv + hkv) << bs_log2) + (uint32_t)(key & ((1 << bs_log2) - 1));
      } else {
        row = (uint32_t)key;
      }
      uint32_t off = (row * D + dma_elem[i]) * 2 + dead;
      // checked build, site 1: a live load's chunk inside the resource (else it moves nothing)
      off = ATTN_IN(dead != 0u || (uint64_t)off + 16 <= kv_bytes, 1) ? off : kDeadOffset;
      ATTN_LDS void* lk = (ATTN_LDS void*)(stage + (i * NW + wave) * 512);
      ATTN_LDS void* lv = (ATTN_LDS void*)(vstage + (i * NW + wave) * 512);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, lk, 16, (int)off, 0, 0, kLoadAux);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, lv, 16, (int)off, 0, 0, kLoadAux);
    }
  };
  auto stage_of = [&](auto s_c) -> uint16_t* {
    constexpr int S = decltype(s_c)::value;
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2;
    else return st3;
  };
  auto vstage_of = [&](auto s_c) -> uint16_t* {
    constexpr int S = decltype(s_c)::value;
    if constexpr (S == 0) return sv0;
    else if constexpr (S == 1) return sv1;
    else if constexpr (S == 2) return sv2;
    else return sv3;
  };

  // ---- query fragments (hi/lo bf16), rotated at q_pos[b] and scaled by log2(e)/sqrt(D); the
  // first tiles' loads go out while the query is read and rotated ----
  const bool qvalid = i16 < Gs;
  int pos = 0;
  if constexpr (ROPE) {
    pos = q_pos[b];
    if (pos < 0 || pos >= table_max_pos) pos = 0;  // such rows are written as NaN at the end
  }
  u32x4 qw[KS];
  f32x4 qc[ROPE ? KS : 1][2];
  {
    const uint16_t* qp = q + ((int64_t)b * Hq + (qvalid ? h0 + i16 : hkv * G)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 32 * ks + 8 * g16;
      qw[ks] = *reinterpret_cast<const u32x4*>(qp + d0);
      if constexpr (ROPE) {
        const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)pos * (D / 2) + d0 / 2);
        qc[ks][0] = tp[0];
        qc[ks][1] = tp[1];
      }
    }
  }
  int ids_a[4] = {0, 0, 0, 0}, ids_b[4] = {0, 0, 0, 0}, ids_c[4] = {0, 0, 0, 0};
  tile_blocks(0, ids_a);
  tile_blocks(1, ids_b);
  tile_blocks(2, ids_c);
  issue(0, st0, sv0, ids_a);
  issue(1, st1, sv1, ids_b);
  issue(2, st2, sv2, ids_c);
  int nid[4] = {0, 0, 0, 0};  // paged: blocks of the next tile to issue
  tile_blocks(kStages - 1, nid);
  bf16x8 qhi[KS], qlo[KS];
  {
    const float qscale = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w = qvalid ? qw[ks] : u32x4{0, 0, 0, 0};
      float x[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) { x[2 * t] = bf16lo(w[t]); x[2 * t + 1] = bf16hi(w[t]); }
      if constexpr (ROPE) {
        const float cs[8] = {qc[ks][0][0], qc[ks][0][1], qc[ks][0][2], qc[ks][0][3],
                             qc[ks][1][0], qc[ks][1][1], qc[ks][1][2], qc[ks][1][3]};
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

  // Per-lane LDS operand offsets (elements) inside this wave's 32-key half.  K (A operand, one
  // ds_read_b128): row 16 kb + i16, logical chunk 4 ks + g16.  V^T (ds_read_b64_tr_b16): row
  // 16 tg + 4 g16 + i16 / 4, logical chunk 2 db + (i16 & 3) / 2, half-chunk i16 & 1.  The
  // swizzle sees only the low row bits, which the half offset (32 rows) does not change.
  int kaddr[2][KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int r = 32 * kw + 16 * kb + i16;
      kaddr[kb][ks] = r * D + swz<D>(r, 4 * ks + g16) * 8;
    }
  int vaddr[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      const int vr = 32 * kw + 16 * tg + 4 * g16 + (i16 >> 2);
      vaddr[db][tg] = vr * D + swz<D>(vr, 2 * db + ((i16 & 3) >> 1)) * 8 + 4 * (i16 & 1);
    }

  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](const uint16_t* stage, const uint16_t* vstage, int t) {
    const int k0 = kbeg + t * kTileKeys + 32 * kw;  // first key of this wave's half
    if (k0 >= kend || k0 + 31 < wstart) return;     // no visible key in it (or past the end)
    const ATTN_LDS uint16_t* sl = (const ATTN_LDS uint16_t*)stage;
    const ATTN_LDS uint16_t* svl = (const ATTN_LDS uint16_t*)vstage;
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 a[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[ks] = *reinterpret_cast<const ATTN_LDS bf16x8*>(sl + kaddr[kb][ks]);
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], qhi[ks], sacc[kb], 0, 0, 0);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], qlo[ks], sacc[kb], 0, 0, 0);
      }
    }
    if (k0 + 32 > kend || k0 < wstart) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + kb * 16 + 4 * g16 + r;
          sacc[kb][r] = (key >= kend || key < wstart) ? -INFINITY : sacc[kb][r];
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
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(sacc[e >> 2][e & 3] - m_run);
      l_run += p;
      pf[e] = (__bf16)p;
    }
    // O^T += V^T P^T ; key order inside the contraction: e -> (e / 4) * 16 + 4 * g16 + e % 4
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 a;
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        const i16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<ATTN_LDS i16x4*>(const_cast<ATTN_LDS uint16_t*>(svl) + vaddr[db][tg]));
        const bf16x4 wb = __builtin_bit_cast(bf16x4, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * tg + e] = wb[e];
      }
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[db], 0, 0, 0);
    }
  };

  // Tile t sits in stage t % 4.  Before it is read, each wave waits for its own loads of it
  // (vmcnt counts this wave's loads in issue order; the two tiles issued after t may stay in
  // flight), then the barrier publishes every wave's part and guarantees every wave is done
  // with tile t - 1, whose stage the loads of tile t + 3 then reuse.  Steps past the last tile
  // (to a multiple of four) only wait, meet the barrier and issue loads that move no data.
  auto step = [&](auto s_c, int t) {
    constexpr int S = decltype(s_c)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((P - 1) * LPT));
    lds_barrier();
    issue(t + P, stage_of(std::integral_constant<int, (S + P) % kStages>{}),
          vstage_of(std::integral_constant<int, (S + P) % kStages>{}), nid);
    compute(stage_of(s_c), vstage_of(s_c), t);
    tile_blocks(t + P + 1, nid);  // paged: their latency passes during the next wait
  };
  for (int t = 0; t < nt; t += kStages) {
    step(std::integral_constant<int, 0>{}, t);
    step(std::integral_constant<int, 1>{}, t + 1);
    step(std::integral_constant<int, 2>{}, t + 2);
    step(std::integral_constant<int, 3>{}, t + 3);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the loads past the end may still write LDS

  // ---- merge the two key halves of each head group ----
  l_run = sum_xor32(sum_xor16(l_run));
  lds_barrier();  // every wave is done reading the stages
  // the partner's O of head group hg in the first two K stages, two head groups each: [DB][4][64]
  // floats (16 x D); the partners' (m, l) in the first V stage: [HG][16][2]
  float* red_o = reinterpret_cast<float*>(hg < 2 ? st0 : st1) + (hg & 1) * 16 * D;
  float (*red_ml)[16][2] = reinterpret_cast<float (*)[16][2]>(sv0);
  if (kw == 1) {
    if (lane < 16) {
      red_ml[hg][i16][0] = m_run;
      red_ml[hg][i16][1] = l_run;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[(db * 4 + r) * 64 + lane] = oacc[db][r];
  }
  lds_barrier();
  if (kw == 1 || Gs <= 0) return;
  const float m1 = red_ml[hg][i16][0], l1 = red_ml[hg][i16][1];
  const float M = fmaxf(m_run, m1);
  const float s0 = M == -INFINITY ? 0.f : fast_exp2(m_run - M);
  const float s1 = M == -INFINITY ? 0.f : fast_exp2(m1 - M);
  const float Lsum = l_run * s0 + l1 * s1;
  const bool valid = qvalid && ATTN_IN(h0 + i16 < Hq, 3);  // checked build, site 3: the output row
  const int h = h0 + i16;
  if constexpr (WHOLE) {
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    float ls = Lsum > 0.f ? (M + log2f(Lsum)) * 0.6931471805599453f : -INFINITY;
    bool bad = false;
    if constexpr (ROPE) {
      const int p = q_pos[b];
      bad = p < 0 || p >= table_max_pos;
      if (bad) ls = __builtin_nanf("");
    }
    if (valid) {
      const int64_t ob = ((int64_t)b * Hq + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = (oacc[db][r] * s0 + red_o[(db * 4 + r) * 64 + lane] * s1) * inv;
          v[r] = bad ? __builtin_nanf("") : x;
        }
        const int d = db * 16 + 4 * g16;
        if constexpr (OUT_BF16) {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(o) + ob + d) =
              u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        } else {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + ob + d) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
      if (lse && g16 == 0) lse[(int64_t)b * Hq + h] = ls;
    }
  } else {
    if (valid) {
      const int64_t part = ((int64_t)b * Hq + h) * n_split + split;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = oacc[db][r] * s0 + red_o[(db * 4 + r) * 64 + lane] * s1;
        *reinterpret_cast<f32x4*>(ws_o + part * D + db * 16 + 4 * g16) = v;
      }
      if (g16 == 0) {
        ws_ml[part * 2 + 0] = M;
        ws_ml[part * 2 + 1] = Lsum;
      }
    }
  }
}

template <int D, bool ROPE, int HG, bool PAGED, bool WIN>
hipError_t go(const DecodeArgs& a, hipStream_t st) {
  const int n_sub = (a.Hq / a.Hkv + 15) / 16;
  const int n_super = (n_sub + HG - 1) / HG;
  const int64_t n_units = (int64_t)a.n_split * a.Hkv * a.B;
  const dim3 grid((unsigned)(((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * n_super));
  const dim3 block(2 * HG * 64);
  const uint16_t* q = (const uint16_t*)a.q;
  const uint16_t* kc = (const uint16_t*)a.k;
  const uint16_t* vc = (const uint16_t*)a.v;
  const float2* tab = reinterpret_cast<const float2*>(a.table);
  auto launch = [&](auto kernel, int n_split) {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, q, kc, vc, a.cache_len, a.q_pos, a.B, a.Hq, a.Hkv, a.S_max, tab,
                       a.table_max_pos, n_split, a.chunk, a.ws_o, a.ws_ml, a.o, a.lse, a.block_table, a.max_blocks,
                       a.bs_log2, a.num_blocks, a.window);
    return hipGetLastError();
  };
  if (a.n_split == 1) {
    return a.out_bf16 ? launch(decode_wide_kernel<D, ROPE, HG, true, true, PAGED, WIN>, 1)
                      : launch(decode_wide_kernel<D, ROPE, HG, true, false, PAGED, WIN>, 1);
  }
  const hipError_t e = launch(decode_wide_kernel<D, ROPE, HG, false, false, PAGED, WIN>, a.n_split);
  if (e != hipSuccess) return e;
  return launch_decode_merge(a, st);
}

template <int D, bool ROPE, bool PAGED>
hipError_t go_hg(const DecodeArgs& a, hipStream_t st) {
  const bool win = a.window < kNoWindow;
  if (a.Hq / a.Hkv <= 32)
    return win ? go<D, ROPE, 2, PAGED, true>(a, st) : go<D, ROPE, 2, PAGED, false>(a, st);
  return win ? go<D, ROPE, 4, PAGED, true>(a, st) : go<D, ROPE, 4, PAGED, false>(a, st);
}

template <bool PAGED>
hipError_t go_d(const DecodeArgs& a, hipStream_t st) {
  const bool rope = a.table != nullptr;
  if (a.D == 64) return rope ? go_hg<64, true, PAGED>(a, st) : go_hg<64, false, PAGED>(a, st);
  return rope ? go_hg<128, true, PAGED>(a, st) : go_hg<128, false, PAGED>(a, st);
}

}  // namespace

ATTN_CHECK_READER(checked_word_decode_wide)

bool decode_wide_fits(const DecodeArgs& a) {
  if (a.Hq / a.Hkv <= 16) return false;
  const int64_t bytes = a.block_table ? (int64_t)a.num_blocks * a.Hkv * ((int64_t)a.D << a.bs_log2) * 2
                                      : (int64_t)a.S_max * a.D * 2;
  return bytes <= kMaxWideBytes;
}

hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t st) {
  return a.block_table ? go_d<true>(a, st) : go_d<false>(a, st);
}

}  // namespace attn
