// bf16 prefill on the gfx950 matrix cores: exact attention tiled with an online softmax.
//
// Method: scaled dot-product attention, devthesis.com "Transformer Architecture & Self-Attention
// Mechanics" section 1; causal mask of the learnllm.online listing; RoPE of devthesis section 3;
// the tiling with a running row max and row sum of codingpancake.com "Building Self-Attention and
// Transformer Engines" sections 4.1-4.2 (the score tile never leaves registers); GQA head sharing
// of the same page, section 6.1.
//
// Shape of the kernel (one workgroup = 4 waves = 128 query rows of one head, two workgroups per
// CU):
//  * Each wave owns 32 query rows.  Its Q rows sit in registers as the B operand of a 32x32x16
//    MFMA: rotated in fp32, scaled by log2(e)/sqrt(D) and rounded to fp16 when RoPE is on; raw
//    bf16 (exact) when it is off.  fp16 rows (queries and keys) that would reach 2^15 are scaled
//    by a power of two first (f16_row_exponent), and the scores of tiles holding such rows are
//    scaled back in fp32; each workgroup checks its key range once and runs a key loop without
//    that test when no row there is scaled.
//  * Keys arrive in tiles of 64, double-buffered in LDS with an XOR swizzle of 16-byte chunks
//    (bank-conflict-free operand reads).  Three ways to fill the K tile:
//      KMODE_PREROT  keys already rotated to fp16 by a one-pass kernel (workspace given): K and V
//                    tiles go HBM -> LDS with no register staging (buffer loads to LDS; the
//                    tail tile with global_load_lds_dwordx4);
//      KMODE_FUSED   RoPE fused into the K tile load: bf16 K and the coefficient rows are staged
//                    in registers, rotated in fp32, stored to LDS as fp16;
//      KMODE_RAW     no RoPE: bf16 K straight to LDS; Q.K^T on bf16 operands (exact products),
//                    the scale folded into the exponent.
//    V always goes HBM -> LDS directly.
//  * Scores are computed transposed, S^T = K Q^T, so that each lane holds 32 scores of ONE query
//    row (the other 32 of the tile sit in lane l^32): the row max is a local max3 tree plus one
//    v_permlane32_swap; the row sum stays lane-local until the end.
//  * P (bf16) is consumed straight from those registers as the B operand of O^T += V^T P^T; the
//    V^T operand comes from LDS through ds_read_b64_tr_b16.  The key order inside the contraction
//    is permuted so that no register shuffle is needed.
//  * Online softmax in log2 units with lazy rescaling: O and l are rescaled only when a row's max
//    grows by more than 8 (unnormalised weights stay <= 2^8); normalised once at the end.
//  * Causal: tiles entirely above a wave's rows are skipped; only tiles crossing the diagonal (or
//    the tail of the keys) are masked.  The diagonal may be shifted by coff keys: a chunk of
//    queries at the end of a longer key sequence (a KV cache) sees every earlier key.
//  * Sliding window (codingpancake.com section 6.4): a query sees only the `window` keys before
//    it (and itself); tiles entirely before a wave's windows are skipped, and the workgroup
//    starts at the first tile any of its rows can see.
//  * Workgroup order: heaviest query blocks first; the G query heads sharing one KV head (and the
//    same query block) go to the same XCD so its L2 serves their K/V reads.
#include "common.h"

namespace attn {

namespace {

constexpr int kWavesStream = 4;            // waves per workgroup
constexpr int kRowsPerWave = 32;
constexpr int kBN = 64;                     // keys per tile
constexpr float kRescaleThreshold = 8.0f;   // log2 units
constexpr float kWeightSumBound = 1024.0f;  // per-lane weight sum that forces a max update
constexpr int kNumXcd = 8;
constexpr int kWaitVmcnt0 = 0x0F70;          // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15)
constexpr int kBufferWord3 = 0x00020000;     // buffer resource word 3: 32-bit data format, raw
constexpr bool kOffsetInit = true;          // scores come out of the MFMA already offset by -m

enum { KMODE_PREROT = 0, KMODE_FUSED = 1, KMODE_RAW = 2 };

// Physical 16-byte chunk of logical chunk `lc` in LDS row `r` (an involution in lc).
template <int D>
__device__ __forceinline__ int swz(int r, int lc) {
  if constexpr (D == 128) {
    return lc ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    return lc ^ (r & 7);
  }
}

// WIN: a sliding window is applied (causal only); without it the window code is compiled out.
// VARPOS: chunks at per-sequence positions (causal only): sequence b's chunk starts at key row
// p = pos0_dev[b], so its keys are rows [0, p + Sq), query row i sees key j <= i + p and sits at
// RoPE position p + i; coff_in is the largest start allowed (the key rows the buffers hold).  A
// start outside [0, coff_in] makes the workgroup write NaN rows instead of reading anything.
template <int D, bool CAUSAL, int KMODE, bool OUT_BF16, int NW, bool WIN, bool VARPOS>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(NW / 2, NW / 2)))
void prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, void* __restrict__ o,
                         float* __restrict__ lse, int B, int Hq, int Hkv, int Sq, int Sk_in,
                         int k_rows, int v_rows, int coff_in, int window, int pos0_in,
                         const float2* __restrict__ table, const uint8_t* __restrict__ kexp,
                         const int32_t* __restrict__ pos0_dev) {
  constexpr int NT = NW * 64;                // threads per workgroup
  constexpr int NCH = D / 8;                 // 16-byte chunks per row
  constexpr int KS = D / 16;                 // MFMA k-steps over D
  constexpr int DB = D / 32;                 // 32-wide output blocks over D
  constexpr int TILE_ELEMS = kBN * D;
  constexpr int DIRECT_PER_WAVE = TILE_ELEMS * 2 / 1024 / NW;  // 1 KB wave-loads per tensor
  constexpr int CPT = kBN * NCH / NT;        // K chunks per thread (fused mode)
  constexpr bool QK_BF16 = KMODE == KMODE_RAW;
  constexpr int BM = NW * kRowsPerWave;      // query rows per workgroup
  static_assert(DIRECT_PER_WAVE * 1024 * NW == TILE_ELEMS * 2, "tile split over waves");
  static_assert(CPT * NT == kBN * NCH, "fused tile split over threads");

  // Two stages, as four distinct LDS objects: with the stage fixed at compile time (the key loop
  // is unrolled by two) the compiler can see that the HBM->LDS loads of the next tile never
  // alias the current tile's operand reads, so it does not wait for them before reading.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[TILE_ELEMS];
  // fused mode, per stage: the exponent byte of each key row of the K tile (f16_row_exponent),
  // and one byte per wave, set when some row it rotated has a non-zero exponent
  __shared__ uint8_t e_lds[KMODE == KMODE_FUSED ? 2 : 1][KMODE == KMODE_FUSED ? kBN : 1];
  __shared__ uint32_t e_flag[KMODE == KMODE_FUSED ? 2 : 1];
  static_assert(KMODE != KMODE_FUSED || NW == 4, "one flag byte per wave, read as one word");

  // ---- workgroup -> (query block, batch, head) ----
  const int G = Hq / Hkv;
  const int nqb = (Sq + BM - 1) / BM;
  const int NG = nqb * B * Hkv;
  const int id = blockIdx.x;
  const int xcd = id % kNumXcd;
  const int j = id / kNumXcd;
  const int gi = (j / G) * kNumXcd + xcd;
  if (gi >= NG) return;
  const int gq = j % G;
  const int qblock = CAUSAL ? (nqb - 1 - gi / (B * Hkv)) : (gi / (B * Hkv));
  const int rem = gi % (B * Hkv);
  const int b = rem / Hkv;
  const int hkv = rem % Hkv;
  const int h = hkv * G + gq;
  int Sk = Sk_in, coff = coff_in, pos0 = pos0_in;
  if constexpr (VARPOS) {
    if (!ATTN_IN(b < B, 0)) return;  // checked build, site 0: the sequence whose start is read
    const int p = __builtin_amdgcn_readfirstlane(pos0_dev[b]);
    if (p < 0 || p > coff_in) {
      // no valid chunk position: the workgroup's output rows (and LSE) become NaN
      const int r0 = qblock * BM, nr = min(BM, Sq - r0);
      const int64_t obase = (((int64_t)b * Hq + h) * Sq + r0) * D;
      for (int i = threadIdx.x; i < nr * D; i += NT) {
        if constexpr (OUT_BF16)
          reinterpret_cast<__bf16*>(o)[obase + i] = (__bf16)__builtin_nanf("");
        else
          reinterpret_cast<float*>(o)[obase + i] = __builtin_nanf("");
      }
      if (lse)
        for (int i = threadIdx.x; i < nr; i += NT) lse[((int64_t)b * Hq + h) * Sq + r0 + i] = __builtin_nanf("");
      return;
    }
    Sk = p + Sq;
    coff = p;
    pos0 = p;
  }
  // checked build, site 0: the workgroup's (batch, head, query block) and the key row counts
  if (!ATTN_IN(b < B && h < Hq && hkv < Hkv && qblock * BM < Sq && Sk >= 1 && Sk <= k_rows && Sk <= v_rows, 0))
    return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int hl = lane >> 5;      // which half of the wave
  const int l32 = lane & 31;
  const int g16 = lane >> 4;     // 16-lane group
  const int i16 = lane & 15;
  const int q0 = qblock * BM;
  const int qw = q0 + wave * kRowsPerWave;  // first row of this wave
  const int row = qw + l32;                 // this lane's query row
  // exp2 argument scale: folded into Q (fp16 modes) or applied to raw scores (bf16 mode)
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);

  // ---- Q fragments (B operand) ----
  typedef typename std::conditional<QK_BF16, bf16x8, f16x8>::type qk_t;
  qk_t qf[KS];

  // ---- key range ----
  // Query row i sees key j when i + coff - window <= j <= i + coff (coff = 0: the square mask;
  // coff = Sk - Sq: the mask aligned at the bottom right, for a chunk of queries at the end of
  // the keys; window >= 2^30: no window).
  const int q_last = min(q0 + BM, Sq) - 1;
  const int key_end = CAUSAL ? min(q_last + 1 + coff, Sk) : Sk;
  const int n_tiles = (key_end + kBN - 1) / kBN;
  const int t_first = (CAUSAL && WIN) ? max(0, q0 + coff - window) / kBN : 0;
  const uint16_t* kg = k + ((int64_t)b * Hkv + hkv) * k_rows * D;
  const uint16_t* vg = v + ((int64_t)b * Hkv + hkv) * v_rows * D;
  // HBM -> LDS with no register staging: wave-load i of this wave fills LDS chunks
  // [(i * NW + wave) * 64, +64); lane L's chunk P holds logical chunk swz(row, P % NCH)
  // of row P / NCH.  The per-lane element offsets are fixed for the whole kernel; each tile adds
  // a wave-uniform base.  Rows past Sk read row Sk-1 (finite data; those keys are masked).
  // Byte offsets are unsigned 32-bit so the loads use the scalar-base + vector-offset form.
  // Wave-load i of this wave fills LDS chunks [(i * NW + wave) * 64, +64): lane L's chunk P holds
  // logical chunk swz(row, P % NCH) of row P / NCH.  Row r_i = r_0 + i * rows_per_load, and the
  // swizzle sees only the low rows bits that i leaves unchanged, so the byte offset of load i is
  // dma_base + i * load_bytes (passed as the load's scalar offset).  Rows past Sk (tail tile only)
  // read row Sk-1 (finite data; those keys are masked).
  constexpr int ROWS_PER_LOAD = NW * 64 / NCH;          // rows one round of wave-loads covers
  constexpr uint32_t LOAD_BYTES = ROWS_PER_LOAD * D * 2;
  static_assert(ROWS_PER_LOAD % 16 == 0 || (D == 64 && ROWS_PER_LOAD % 8 == 0), "swizzle period");
  const int dma_r0 = (wave * 64 + lane) / NCH;
  const uint32_t dma_base = (uint32_t)(dma_r0 * D + swz<D>(dma_r0, (wave * 64 + lane) % NCH) * 8) * 2u;
  auto direct_tile = [&](const uint16_t* src, uint16_t* dst_tile, int k0) {
    const char* base = reinterpret_cast<const char*>(src + (int64_t)k0 * D);
    if (k0 + kBN <= Sk) {
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, kBN * D * 2, kBufferWord3);
#pragma unroll
      for (int i = 0; i < DIRECT_PER_WAVE; ++i) {
        ATTN_LDS void* l = (ATTN_LDS void*)(dst_tile + (i * NW + wave) * 512);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, l, 16, (int)dma_base, (int)(LOAD_BYTES * i), 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < DIRECT_PER_WAVE; ++i) {
        // (the no-op keeps this address arithmetic in the tail branch: hoisted, it ran every tile)
        int r = dma_r0 + ROWS_PER_LOAD * i;
        asm volatile("" : "+v"(r));
        const int rr = min(r, Sk - 1 - k0);
        uint32_t off = dma_base + LOAD_BYTES * i - (uint32_t)((r - rr) * D * 2);
        // checked build, site 1: the tail tile's source chunk lies within rows [k0, Sk)
        off = ATTN_IN(off + 16 <= (uint32_t)(Sk - k0) * D * 2, 1) ? off : 0u;
        const void* g = base + off;
        ATTN_LDS void* l = (ATTN_LDS void*)(dst_tile + (i * NW + wave) * 512);
        __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
      }
    }
  };
  // Per-lane LDS operand offsets (bytes).  K operand (ds_read_b128): row kb*32 + l32, logical
  // chunk 2*ks + hl.  V^T operand (ds_read_b64_tr_b16): row kb*32 + 16*s + 8*tg + 4*hl + i16/4,
  // logical chunk 4*db + 2*(g16&1) + (i16&3)/2, half-chunk i16&1.  The swizzle only sees the low
  // four row bits, which kb and s do not change, so those enter as immediate offsets.
  int kaddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kaddr[ks] = (l32 * D + swz<D>(l32, 2 * ks + hl) * 8) * 2;
    // checked build, site 2: both 32-key blocks' operands inside the tile
    kaddr[ks] = ATTN_IN(kaddr[ks] >= 0 && kaddr[ks] + 32 * D * 2 + 16 <= TILE_ELEMS * 2, 2) ? kaddr[ks] : 0;
  }
  int vaddr[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      const int vr = 8 * tg + 4 * hl + (i16 >> 2);
      const int lc = 4 * db + 2 * (g16 & 1) + ((i16 & 3) >> 1);
      vaddr[db][tg] = (vr * D + swz<D>(vr, lc) * 8 + 4 * (i16 & 1)) * 2;
      // checked build, site 2: the farthest row the reads add (48 rows on) inside the tile
      vaddr[db][tg] = ATTN_IN(vaddr[db][tg] >= 0 && vaddr[db][tg] + 48 * D * 2 + 8 <= TILE_ELEMS * 2, 2)
                          ? vaddr[db][tg] : 0;
    }

  // fused-mode staging (bf16 K + its coefficient rows)
  u32x4 kst[KMODE == KMODE_FUSED ? CPT : 1];
  f32x4 tst[KMODE == KMODE_FUSED ? CPT : 1][2];
  auto fused_issue = [&](int k0) {
    if constexpr (KMODE == KMODE_FUSED) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + NT * i;
        const int r = c / NCH, cc = c % NCH;
        int key = min(k0 + r, Sk - 1);
        key = ATTN_IN(key >= 0 && key < k_rows && cc < NCH, 3) ? key : 0;  // checked build, site 3
        kst[i] = *reinterpret_cast<const u32x4*>(kg + (int64_t)key * D + cc * 8);
        const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)(pos0 + key) * (D / 2) + cc * 4);
        tst[i][0] = tp[0];
        tst[i][1] = tp[1];
      }
    }
  };
  auto fused_store = [&](uint16_t* k_tile) {
    if constexpr (KMODE == KMODE_FUSED) {
      bool wave_big = false;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + NT * i;
        const int r = c / NCH, cc = c % NCH;
        float x[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) { x[2 * t] = bf16lo(kst[i][t]); x[2 * t + 1] = bf16hi(kst[i][t]); }
        const float cs[8] = {tst[i][0][0], tst[i][0][1], tst[i][0][2], tst[i][0][3],
                             tst[i][1][0], tst[i][1][1], tst[i][1][2], tst[i][1][3]};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float c = cs[2 * p], s = cs[2 * p + 1];
          const float x0 = x[2 * p], x1 = x[2 * p + 1];
          x[2 * p] = x0 * c - x1 * s;
          x[2 * p + 1] = x0 * s + x1 * c;
        }
        // The row's exponent: its NCH chunks are held by NCH consecutive lanes.  Rows below 2^15
        // (every row, in practice) are packed as they are; only a wave holding a larger element
        // finds the exponents of its rows.
        const float mx = fmaxf(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))),
                               fmaxf(fmaxf(fabsf(x[4]), fabsf(x[5])), fmaxf(fabsf(x[6]), fabsf(x[7]))));
        int e = 0;
        if (__builtin_amdgcn_ballot_w64(!(mx < 32768.f)) != 0) {
          e = f16_row_exponent(group_max<NCH>(mx));
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = ldexpf(x[t], -e);
          wave_big = true;
        }
        u32x4 kh;
#pragma unroll
        for (int t = 0; t < 4; ++t) kh[t] = pack_f16(x[2 * t], x[2 * t + 1]);
        const int off = r * D + swz<D>(r, cc) * 8;
        *reinterpret_cast<ATTN_LDS u32x4*>((ATTN_LDS uint16_t*)(k_tile) + off) = kh;
        if (cc == 0) e_lds[k_tile == k_lds0 ? 0 : 1][r] = (uint8_t)e;
      }
      if (lane == 0) reinterpret_cast<uint8_t*>(&e_flag[k_tile == k_lds0 ? 0 : 1])[wave] = wave_big ? 1 : 0;
    }
  };
  auto issue_tile = [&](int k0, uint16_t* k_tile, uint16_t* v_tile) {
    if constexpr (KMODE != KMODE_FUSED) direct_tile(kg, k_tile, k0);
    direct_tile(vg, v_tile, k0);
  };

  // ---- accumulators ----
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running row max of the exp2-domain scores
  float l_run = 0.f;        // this lane's half of the row sum
  // Offset the score MFMA starts from: -m_run once m_run is finite (the scores then come out as
  // s - m_run and need no subtraction); 0 before the first tile.  The pre-rotated and raw modes
  // keep it as a block of 16 registers across the key loop.  The fused mode, whose K staging
  // registers leave no room for that block (it spilled 7-8 registers), writes it into the score
  // accumulators at the start of each tile instead (16 moves per tile, +4.6% measured there;
  // neutral to -1% in the other modes).
  constexpr bool kOffsetPerTile = KMODE == KMODE_FUSED;
  float s_init = 0.f;
  f32x16 s_init_v;
#pragma unroll
  for (int r = 0; r < 16; ++r) s_init_v[r] = 0.f;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // Row exponents of the fp16 operands (f16_row_exponent): qa of this lane's query row (q_scaled:
  // some row of the wave has one), and the exponent byte of key row k0 + lane of the current tile
  // (pre-rotated keys: loaded one tile ahead with the tile's loads).  A tile where any of them is
  // non-zero forms its products from 0 and scales them, s - m = 2^(qa + e) q'.k' + s_init, which is
  // as accurate as starting the products from s_init; other tiles take the usual path.
  constexpr bool EXPS = !QK_BF16;
  int qa = 0;
  bool q_scaled = false;
  int e_cur = 0, e_next = 0;
  const uint8_t* kexp_head = kexp ? kexp + ((int64_t)b * Hkv + hkv) * k_rows : nullptr;
  auto load_exps = [&](int k0) {
    if constexpr (KMODE == KMODE_PREROT) e_next = kexp_head[min(k0 + lane, Sk - 1)];
  };

  // One key tile: t is the tile index; the stage (and so every LDS address) is fixed at compile
  // time by STAGE.
  auto tile_step = [&](auto stage_c, auto scaled_c, int t) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr bool SCALED = decltype(scaled_c)::value;
    uint16_t* k_cur = STAGE ? k_lds1 : k_lds0;
    uint16_t* v_cur = STAGE ? v_lds1 : v_lds0;
    uint16_t* k_nxt = STAGE ? k_lds0 : k_lds1;
    uint16_t* v_nxt = STAGE ? v_lds0 : v_lds1;
    const int k0 = t * kBN;
    fused_store(k_cur);
    // Each wave drains its own HBM->LDS loads of tile t (vmcnt is per wave), then the barrier
    // makes every wave's part visible and guarantees every wave is done with tile t-1.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if constexpr (SCALED && KMODE == KMODE_PREROT) e_cur = e_next;
    if (t + 1 < n_tiles) {
      issue_tile(k0 + kBN, k_nxt, v_nxt);
      if constexpr (SCALED) load_exps(k0 + kBN);
    }

    if (!CAUSAL || (k0 <= qw + kRowsPerWave - 1 + coff && (!WIN || k0 + kBN - 1 >= qw + coff - window))) {
      const ATTN_LDS uint16_t* kb_lds = (const ATTN_LDS uint16_t*)(k_cur);
      const ATTN_LDS uint16_t* vb_lds = (const ATTN_LDS uint16_t*)(v_cur);
      // S^T = K Q^T for two 32-key blocks, the products of each starting from c0
      f32x16 sacc[2];
      auto scores = [&](const f32x16& c0) __attribute__((always_inline)) {
        if constexpr (kOffsetPerTile) {
          // the two blocks' k-steps interleaved, operand reads two steps (four reads) ahead of
          // the MFMAs that use them (+1.8% in the fused mode, neutral in the others)
          qk_t a[2][KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              a[kb][ks] = *reinterpret_cast<const ATTN_LDS qk_t*>((const ATTN_LDS char*)kb_lds + kaddr[ks] +
                                                                  kb * 32 * D * 2);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[kb][ks], qf[ks], ks == 0 ? c0 : sacc[kb], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // 0x100: LDS reads
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); // 0x008: MFMAs
            if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            qk_t a[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              a[ks] = *reinterpret_cast<const ATTN_LDS qk_t*>((const ATTN_LDS char*)kb_lds + kaddr[ks] + kb * 32 * D * 2);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const f32x16 c = ks == 0 ? c0 : sacc[kb];
              if constexpr (QK_BF16)
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[ks], c, 0, 0, 0);
              else
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks], qf[ks], c, 0, 0, 0);
            }
          }
        }
      };
      // key exponents of the tile: pre-rotated keys hold row k0 + lane's in e_cur; fused RoPE
      // reads them from e_lds (the stage's bytes stay put until the next barrier)
      auto key_exp = [&](int key) __attribute__((always_inline)) {
        if constexpr (KMODE == KMODE_FUSED) return (int)e_lds[STAGE][key];
        else return __builtin_amdgcn_ds_bpermute(key << 2, e_cur);
      };
      bool scaled_tile = false;
      if constexpr (SCALED) {
        if constexpr (KMODE == KMODE_FUSED)
          scaled_tile = q_scaled || e_flag[STAGE] != 0;
        else
          scaled_tile = q_scaled || __builtin_amdgcn_ballot_w64(e_cur != 0) != 0;
      }
      // Scaled rows present (rare): the products start from 0 and become 2^(qa + e) q'.k' +
      // s_init, with e the exponent of each score's key.  The offset block is cleared for the one
      // score pass and restored afterwards, inside branches (the empty asm keeps the compiler from
      // turning them into a select of every element on every tile).
      if constexpr (kOffsetPerTile) {
        // the empty asm makes the offset a new value on every tile, so the compiler writes it
        // into the accumulators instead of keeping a copy live across the loop
        float si = scaled_tile ? 0.f : s_init;
        asm volatile("" : "+v"(si));
        f32x16 c0;
#pragma unroll
        for (int r = 0; r < 16; ++r) c0[r] = si;
        scores(c0);
      } else {
        if (scaled_tile) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s_init_v[r] = 0.f;
          asm volatile("");
        }
        // the first product starts from the offset block (s_init in every element)
        scores(s_init_v);
      }
      if (scaled_tile) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ek = key_exp(kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3));
            sacc[kb][r] = ldexpf(sacc[kb][r], qa + ek) + s_init;
          }
        if constexpr (!kOffsetPerTile) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s_init_v[r] = s_init;
          asm volatile("");
        }
      }
      if constexpr (QK_BF16) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] *= c_log2;
      }
      // mask (diagonal / tail tiles only)
      const bool need_mask =
          (CAUSAL && (k0 + kBN - 1 > qw + coff || (WIN && k0 < qw + kRowsPerWave - 1 + coff - window))) ||
          (k0 + kBN > Sk);
      if (need_mask) {
        // score (kb, r) belongs to key k0 + 4*hl + c with c = kb*32 + 8*(r>>2) + (r&3) fixed at
        // compile time: it is visible when lo <= c <= hi, two bounds per lane
        const int base = k0 + 4 * hl;
        int hi = Sk - 1 - base;
        if constexpr (CAUSAL) hi = min(hi, row + coff - base);
        const int lo = (CAUSAL && WIN) ? row + coff - window - base : 0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
            if (c > hi || (CAUSAL && WIN && c < lo)) sacc[kb][r] = -INFINITY;
          }
      }
      bf16x8 pf[2][2];
      float lsum = 0.f;
      // p = 2^score rounded to bf16 (the B operand of P.V); the row sum adds the same rounded
      // weights, two at a time (v_dot2_f32_bf16 against (1, 1)), in two independent chains
      auto weights = [&]() __attribute__((always_inline)) {
        float ls[2] = {0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int tt = 0; tt < 8; tt += 2) {
              bf16x2 pp;
              pp[0] = (__bf16)fast_exp2(sacc[kb][8 * s + tt]);
              pp[1] = (__bf16)fast_exp2(sacc[kb][8 * s + tt + 1]);
              pf[kb][s][tt] = pp[0];
              pf[kb][s][tt + 1] = pp[1];
              ls[kb] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls[kb], false);
            }
        lsum = ls[0] + ls[1];
      };
      auto tile_max = [&]() __attribute__((always_inline)) {
        float mx = sacc[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
        return fmaxf(mx, swap_halves(mx));
      };
      if constexpr (kOffsetInit && !QK_BF16) {
        // sacc = s - m_run (s itself while m_run is -inf).  The weights are formed directly; the
        // tile max is taken only when this lane's weight sum leaves [0, kWeightSumBound] (some
        // score rose well above m_run; the first tile, where m_run is -inf, always does).  Then O
        // and l move to the tile max and the weights are formed again.  Without that, every
        // weight is at most kWeightSumBound, so O and l stay far from overflow.
        weights();
        if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY || !(lsum <= kWeightSumBound)) != 0) {
          const float mx = tile_max();
          const float m_new = m_run == -INFINITY ? mx : m_run + fmaxf(mx, 0.f);
          // none: the row has seen no key yet (only with a sliding window); it stays at -inf
          const bool none = WIN && m_new == -INFINITY;
          const float alpha = none ? 1.f : fast_exp2(m_run - m_new);   // 0 while m_run is -inf
          const float shift = none ? 0.f : m_new + s_init;   // subtract to put sacc on m_new's scale
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] -= shift;
          m_run = m_new;
          s_init = none ? 0.f : -m_new;
          if constexpr (!kOffsetPerTile) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s_init_v[r] = s_init;
          }
          weights();
        }
      } else {
        const float mx = tile_max();
        const float m_new = fmaxf(m_run, mx);
        const bool need = m_new > m_run + kRescaleThreshold;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
          // a row that still sees no key (sliding window) keeps m = -inf and needs no rescale
          const float alpha = (WIN && m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          m_run = m_new;
        }
        // p = 2^(s - m), packed to bf16 as the B operand of P.V; the row sum adds the same
        // rounded weights, two at a time (v_dot2_f32_bf16 against (1, 1)).  A row that has seen
        // no key yet (sliding window) has m = -inf and only -inf scores: its weights are 0.
        const float m_sub = (WIN && m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int tt = 0; tt < 8; tt += 2) {
              bf16x2 pp;
              pp[0] = (__bf16)fast_exp2(sacc[kb][8 * s + tt] - m_sub);
              pp[1] = (__bf16)fast_exp2(sacc[kb][8 * s + tt + 1] - m_sub);
              pf[kb][s][tt] = pp[0];
              pf[kb][s][tt + 1] = pp[1];
              lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
            }
      }
      l_run += lsum;
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 va[2][DB];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int tg = 0; tg < 2; ++tg) {
              ATTN_LDS i16x4* pa = reinterpret_cast<ATTN_LDS i16x4*>(
                  (ATTN_LDS char*)(const_cast<ATTN_LDS uint16_t*>(vb_lds)) + vaddr[db][tg] +
                  (kb * 32 + 16 * s) * D * 2);
              const i16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pa);
              const bf16x4 wb = __builtin_bit_cast(bf16x4, w);
#pragma unroll
              for (int e = 0; e < 4; ++e) va[s][db][4 * tg + e] = wb[e];
            }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s][db], pf[kb][s], oacc[db], 0, 0, 0);
      }
    }
    // Fused RoPE: the next tile's keys and coefficients are fetched only now, so the staging
    // registers are not live across the tile's MFMA work (no spills); the other workgroup on the
    // CU covers the load latency.
    if (t + 1 < n_tiles) fused_issue(k0 + kBN);
  };

  // The first tile's loads go out before the Q rows are read and rotated, so the two latencies
  // overlap at the start of every workgroup.
  issue_tile(t_first * kBN, k_lds0, v_lds0);
  fused_issue(t_first * kBN);
  load_exps(t_first * kBN);
  {
    const int rc = row < Sq ? row : Sq - 1;
    const uint16_t* qrow = q + (((int64_t)b * Hq + h) * Sq + rc) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 16 * ks + 8 * hl;
      const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + d0);
      if constexpr (QK_BF16) qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
    if constexpr (!QK_BF16) {
      // the row rotated and scaled by log2(e)/sqrt(D), its exponent, then the row (scaled by 2^-qa
      // when some row of the wave has one) rounded to fp16
      auto rotated = [&](int ks, float (&x)[8]) __attribute__((always_inline)) {
        const int d0 = 16 * ks + 8 * hl;
        const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + d0);
#pragma unroll
        for (int t = 0; t < 4; ++t) { x[2 * t] = bf16lo(w[t]); x[2 * t + 1] = bf16hi(w[t]); }
        const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)(pos0 + rc) * (D / 2) + d0 / 2);
        const f32x4 c01 = tp[0], c23 = tp[1];
        const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float c = cs[2 * p], s = cs[2 * p + 1];
          const float x0 = x[2 * p], x1 = x[2 * p + 1];
          x[2 * p] = (x0 * c - x1 * s) * c_log2;
          x[2 * p + 1] = (x0 * s + x1 * c) * c_log2;
        }
      };
      float xq[KS][8];
      float qmax = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        rotated(ks, xq[ks]);
#pragma unroll
        for (int t = 0; t < 8; ++t) qmax = fmaxf(qmax, fabsf(xq[ks][t]));
      }
      qa = f16_row_exponent(fmaxf(qmax, swap_halves(qmax)));
      q_scaled = __builtin_amdgcn_ballot_w64(qa != 0) != 0;
      if (q_scaled) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int t = 0; t < 8; ++t) xq[ks][t] = ldexpf(xq[ks][t], -qa);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < 8; ++t) qf[ks][t] = (_Float16)xq[ks][t];
    }
  }

  // Which key loop: the scaled one tests every tile for row exponents; the plain one has no such
  // test.  Fused RoPE finds the key exponents only tile by tile, so it always takes the scaled
  // loop; bf16 operands (no RoPE) have none.  Pre-rotated keys: every thread ORs 16-byte words of
  // the exponent bytes covering [t_first * kBN, key_end), and the workgroup takes the scaled loop
  // if any exponent there, or any qa of its rows, is non-zero.  The exponent area starts 16-byte
  // aligned and its size is rounded up to 256 bytes, so the words stay inside it; bytes of
  // neighbouring rows only make the test conservative.
  bool scaled_wg = KMODE == KMODE_FUSED;
  if constexpr (KMODE == KMODE_PREROT) {
    uint32_t acc = q_scaled ? 1u : 0u;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(kexp_head + t_first * kBN) & ~(uintptr_t)15;
    uintptr_t hi = (reinterpret_cast<uintptr_t>(kexp_head + key_end) + 15) & ~(uintptr_t)15;
    // checked build, site 5: the words read lie inside the exponent area (else: no words read,
    // and the workgroup takes the scaled loop, which reads the bytes one by one)
    if (!ATTN_IN(lo >= reinterpret_cast<uintptr_t>(kexp) &&
                     hi <= reinterpret_cast<uintptr_t>(kexp) + ((size_t)B * Hkv * k_rows + 255) / 256 * 256,
                 5)) {
      hi = lo;
      acc = 1u;
    }
    for (uintptr_t p = lo + 16 * (uintptr_t)tid; p < hi; p += 16 * NT) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(p);
      acc |= w[0] | w[1] | w[2] | w[3];
    }
    scaled_wg = __syncthreads_or(acc != 0) != 0;
  }
  auto key_loop = [&](auto scaled_c) __attribute__((always_inline)) {
    for (int t = t_first; t < n_tiles; t += 2) {
      tile_step(std::integral_constant<int, 0>{}, scaled_c, t);
      if (t + 1 < n_tiles) tile_step(std::integral_constant<int, 1>{}, scaled_c, t + 1);
    }
  };
  if constexpr (EXPS) {
    if (scaled_wg)
      key_loop(std::true_type{});
    else
      key_loop(std::false_type{});
  } else {
    key_loop(std::false_type{});
  }

  // ---- finalize ----
  const float l_tot = l_run + swap_halves(l_run);
  // checked build, site 6: the output row
  if (row < Sq && ATTN_IN(row >= 0 && ((int64_t)b * Hq + h) * Sq + row < (int64_t)B * Hq * Sq, 6)) {
    const float inv = 1.0f / l_tot;
    const int64_t orow = (((int64_t)b * Hq + h) * Sq + row) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * hl;
        const float o0 = oacc[db][4 * r4 + 0] * inv, o1 = oacc[db][4 * r4 + 1] * inv;
        const float o2 = oacc[db][4 * r4 + 2] * inv, o3 = oacc[db][4 * r4 + 3] * inv;
        if constexpr (OUT_BF16) {
          u32x2 w;
          w[0] = pack_bf16(o0, o1);
          w[1] = pack_bf16(o2, o3);
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(o) + orow + d0) = w;
        } else {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + orow + d0) = f32x4{o0, o1, o2, o3};
        }
      }
    if (lse && hl == 0) lse[((int64_t)b * Hq + h) * Sq + row] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
  }
}

template <int D, bool CAUSAL, int KMODE, bool OUT_BF16, bool WIN, bool VARPOS = false>
hipError_t go(const PrefillArgs& a, const void* kptr, hipStream_t st) {
  constexpr int NW = kWavesStream;
  constexpr int BM = NW * kRowsPerWave;
  const int G = a.Hq / a.Hkv;
  const int nqb = (a.S + BM - 1) / BM;
  const int64_t NG = (int64_t)nqb * a.B * a.Hkv;
  const int64_t blocks = ((NG + kNumXcd - 1) / kNumXcd) * kNumXcd * G;
  // pre-rotated keys: their exponent bytes follow the fp16 rows (k_rows per batch and KV head)
  const uint8_t* kexp = KMODE == KMODE_PREROT
                            ? static_cast<const uint8_t*>(kptr) + prefill_kexp_offset(a.B, a.Hkv, a.k_rows, D)
                            : nullptr;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, KMODE, OUT_BF16, NW, WIN, VARPOS>), dim3((unsigned)blocks),
                     dim3(NW * 64), 0, st, (const uint16_t*)a.q, (const uint16_t*)kptr,
                     (const uint16_t*)a.v, a.o, a.lse, a.B, a.Hq, a.Hkv, a.S, a.Sk, a.k_rows,
                     a.v_rows, a.coff, a.window, a.pos0, reinterpret_cast<const float2*>(a.table), kexp,
                     a.pos0_dev);
  return hipGetLastError();
}

template <int D, int KMODE>
hipError_t dispatch_mode(const PrefillArgs& a, const void* kptr, hipStream_t st) {
  if (a.causal) {
    if (a.window < kNoWindow)
      return a.out_bf16 ? go<D, true, KMODE, true, true>(a, kptr, st) : go<D, true, KMODE, false, true>(a, kptr, st);
    return a.out_bf16 ? go<D, true, KMODE, true, false>(a, kptr, st) : go<D, true, KMODE, false, false>(a, kptr, st);
  }
  return a.out_bf16 ? go<D, false, KMODE, true, false>(a, kptr, st) : go<D, false, KMODE, false, false>(a, kptr, st);
}

// chunks at per-sequence positions (always causal)
template <int D, int KMODE>
hipError_t dispatch_varpos(const PrefillArgs& a, const void* kptr, hipStream_t st) {
  if (a.window < kNoWindow)
    return a.out_bf16 ? go<D, true, KMODE, true, true, true>(a, kptr, st)
                      : go<D, true, KMODE, false, true, true>(a, kptr, st);
  return a.out_bf16 ? go<D, true, KMODE, true, false, true>(a, kptr, st)
                    : go<D, true, KMODE, false, false, true>(a, kptr, st);
}

template <int D>
hipError_t dispatch_d(const PrefillArgs& a, hipStream_t st) {
  if (!a.table) return dispatch_mode<D, KMODE_RAW>(a, a.k, st);
  if (!a.workspace) return dispatch_mode<D, KMODE_FUSED>(a, a.k, st);
  // one pass: rotated fp16 keys into the workspace, then the attention kernel streams them
  const hipError_t e = launch_rotate_keys_f16(a.k, a.workspace, a.B, a.Hkv, a.S, D, a.pos0, a.table, st);
  if (e != hipSuccess) return e;
  return dispatch_mode<D, KMODE_PREROT>(a, a.workspace, st);
}

}  // namespace

size_t prefill_workspace_bytes(int B, int Hkv, int S, int D) {
  const size_t exps = ((size_t)B * Hkv * S + 255) / 256 * 256;
  return prefill_kexp_offset(B, Hkv, S, D) + exps;
}

ATTN_CHECK_READER(checked_word_prefill_bf16)

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st) {
  return a.D == 64 ? dispatch_d<64>(a, st) : dispatch_d<128>(a, st);
}

hipError_t launch_prefill_prerotated(const PrefillArgs& a, const void* k_rot, hipStream_t st) {
  return a.D == 64 ? dispatch_mode<64, KMODE_PREROT>(a, k_rot, st)
                   : dispatch_mode<128, KMODE_PREROT>(a, k_rot, st);
}

hipError_t launch_prefill_cache(const PrefillArgs& a, hipStream_t st) {
  if (a.pos0_dev) {
    if (a.table)
      return a.D == 64 ? dispatch_varpos<64, KMODE_PREROT>(a, a.k, st) : dispatch_varpos<128, KMODE_PREROT>(a, a.k, st);
    return a.D == 64 ? dispatch_varpos<64, KMODE_RAW>(a, a.k, st) : dispatch_varpos<128, KMODE_RAW>(a, a.k, st);
  }
  if (a.table)
    return a.D == 64 ? dispatch_mode<64, KMODE_PREROT>(a, a.k, st) : dispatch_mode<128, KMODE_PREROT>(a, a.k, st);
  return a.D == 64 ? dispatch_mode<64, KMODE_RAW>(a, a.k, st) : dispatch_mode<128, KMODE_RAW>(a, a.k, st);
}

}  // namespace attn
