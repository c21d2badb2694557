// KV cache maintenance for chunked prefill: a chunk of Sq new tokens at positions
// pos0 .. pos0+Sq-1 is appended to a bf16 cache [B*Hkv, S_max, D].
//
// The cache keeps the keys and values of earlier tokens so that later queries reuse them
// ("Transformer internals: attention without the mysticism", ninaddeshpande.com, "The KV cache
// and the memory wall"); the keys are stored already rotated (RoPE of "Transformer Architecture
// & Self-Attention Mechanics", devthesis.com, section 3), so a key is rotated once, when it is
// appended, at its absolute position.
//
// One pass, HBM-bound, every lane moving 16-byte chunks (coalesced along D):
//  * new rows s in [pos0, pos0+Sq): the key is rotated in fp32 with the table row s and rounded
//    to bf16 (nearest even) into the cache; the value is copied;
//  * with RoPE the attention kernel multiplies fp16 operands, so every key row [0, pos0+Sq) is
//    also written to k16 [B*Hkv, pos0+Sq, D] as fp16: the earlier rows converted from the cache,
//    the new rows from the very bf16 values just stored, each row scaled by 2^-e with its
//    exponent byte e in kexp [B*Hkv, pos0+Sq] (f16_row_exponent: e = 0 unless the row reaches
//    2^15; bf16 -> fp16 is then exact for 6.1e-5 <= |x|, smaller magnitudes round to fp16's
//    subnormal grid, 2^-24).  The NCH lanes of one row are consecutive, so a row's maximum is a
//    group reduction.
//
// Paged cache (cache_append_paged_kernel): the pool [num_blocks, Hkv, bs, D] and block table of
// codingpancake.com "Building Self-Attention and Transformer Engines", section 6.2; token t of
// sequence b sits in block block_table[b][t / bs], slot t % bs.  The new rows go into their
// blocks as above, and every row the attention can read, [conv_first, pos0+Sq), is also gathered
// into contiguous workspace copies: the keys (fp16 with RoPE, bf16 without) and the values
// (bf16), which the attention kernel then streams as it streams a contiguous cache.  Rows before
// first_seen (the first query's window start; no query sees them) are written as zeros instead
// of being read, so blocks wholly before it, and their table entries, are never touched.
//
// Append only (kv_append_kernel): the new rows alone, at per-sequence positions, into either
// cache layout -- the step before a decode in a serving loop.
#include "common.h"

namespace attn {

namespace {

// A key row segment of 8 bf16 values (one lane's 16 bytes) as fp16 scaled by 2^-e, e the exponent
// of the whole row (its NCH lanes together); returns e.
template <int NCH>
__device__ __forceinline__ int to_f16_row(const u32x4 w, u32x4& h) {
  float mx = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) mx = fmaxf(mx, fmaxf(fabsf(bf16lo(w[t])), fabsf(bf16hi(w[t]))));
  const int e = f16_row_exponent(group_max<NCH>(mx));
#pragma unroll
  for (int t = 0; t < 4; ++t) h[t] = pack_f16(ldexpf(bf16lo(w[t]), -e), ldexpf(bf16hi(w[t]), -e));
  return e;
}

// One lane's 16-byte key segment (chunk cc of a row: 4 adjacent pairs) rotated in fp32 at
// position s with the table row s and rounded to bf16 (nearest even).
template <int D>
__device__ __forceinline__ u32x4 rope_chunk_bf16(const u32x4 kw, const float2* __restrict__ table, int s, int cc) {
  const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)s * (D / 2) + cc * 4);
  const f32x4 c01 = tp[0], c23 = tp[1];
  const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
  u32x4 kb;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float x0 = bf16lo(kw[p]), x1 = bf16hi(kw[p]);
    const float c = cs[2 * p], sn = cs[2 * p + 1];
    kb[p] = pack_bf16(x0 * c - x1 * sn, x0 * sn + x1 * c);
  }
  return kb;
}

// VARPOS: chunks at per-sequence positions.  The grid then covers rows [0, pos0 + Sq) of every
// (batch, KV head), pos0 being the largest start allowed and the k16 / kexp row count; sequence
// b's chunk starts at p = pos0_dev[b], and only its rows [p, p + Sq) (with RoPE: from its own
// conv_first, the tile of p - window) are written.  A sequence whose p lies outside [0, pos0]
// is left untouched.
template <int D, bool ROPE, bool VARPOS>
__global__ __launch_bounds__(256) void cache_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, uint16_t* __restrict__ k16,
    uint8_t* __restrict__ kexp, int64_t n_bh, int Sq, int S_max, int pos0_in, int conv_first,
    const float2* __restrict__ table, const int32_t* __restrict__ pos0_dev, int Hkv, int window) {
  constexpr int NCH = D / 8;  // 16-byte chunks per row
  // rows handled per (batch, KV head): [first, pos0 + Sq); with RoPE the earlier rows from
  // conv_first on (those a sliding window can still see) are converted to fp16
  const int first = VARPOS ? 0 : ROPE ? conv_first : pos0_in;
  const int Sk = pos0_in + Sq;  // rows per (batch, KV head) of k16 and kexp
  const int nrows = Sk - first;
  const int64_t n = n_bh * nrows * NCH;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int cc = (int)(idx % NCH);
    const int64_t rr = idx / NCH;
    const int s = first + (int)(rr % nrows);
    const int64_t bh = rr / nrows;
    const int64_t crow = (bh * S_max + s) * D + cc * 8;  // element offset in the cache
    int pos0 = pos0_in;
    if constexpr (VARPOS) {
      // the NCH lanes of a row share s and bh, so they skip together (to_f16_row needs all of them)
      pos0 = pos0_dev[bh / Hkv];
      if (pos0 < 0 || pos0 > pos0_in) continue;
      const int lo = !ROPE ? pos0 : window >= pos0 ? 0 : ((pos0 - window) / 64) * 64;
      if (s < lo || s >= pos0 + Sq) continue;
    }
    // checked build, site 0: the row in the cache, in the fp16 copy and in the chunk
    if (!ATTN_IN(bh < n_bh && s >= 0 && s < Sk && Sk <= S_max && (s < pos0 || s - pos0 < Sq), 0)) continue;
    if (s < pos0) {
      // earlier token (RoPE only): its stored bf16 key, converted to fp16
      const u32x4 w = *reinterpret_cast<const u32x4*>(k_cache + crow);
      u32x4 h;
      const int e = to_f16_row<NCH>(w, h);
      *reinterpret_cast<u32x4*>(k16 + (bh * Sk + s) * D + cc * 8) = h;
      if (cc == 0) kexp[bh * Sk + s] = (uint8_t)e;
      continue;
    }
    const int64_t nrow = (bh * Sq + (s - pos0)) * D + cc * 8;  // element offset in the chunk
    const u32x4 kw = *reinterpret_cast<const u32x4*>(k_new + nrow);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(v_new + nrow);
    if constexpr (ROPE) {
      const u32x4 kb = rope_chunk_bf16<D>(kw, table, s, cc);
      u32x4 kh;
      const int e = to_f16_row<NCH>(kb, kh);
      *reinterpret_cast<u32x4*>(k_cache + crow) = kb;
      *reinterpret_cast<u32x4*>(k16 + (bh * Sk + s) * D + cc * 8) = kh;
      if (cc == 0) kexp[bh * Sk + s] = (uint8_t)e;
    } else {
      *reinterpret_cast<u32x4*>(k_cache + crow) = kw;
    }
    *reinterpret_cast<u32x4*>(v_cache + crow) = vw;
  }
}

template <int D, bool VARPOS>
hipError_t append_go(const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* k16,
                     int B, int Hkv, int Sq, int S_max, int pos0, int conv_first, const float* table,
                     const int32_t* pos0_dev, int window, hipStream_t st) {
  const int64_t n_bh = (int64_t)B * Hkv;
  const int64_t rows = VARPOS ? (int64_t)(pos0 + Sq) : table ? (int64_t)(pos0 + Sq - conv_first) : (int64_t)Sq;
  const int64_t n = n_bh * rows * (D / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 workgroups per CU
  if (blocks < 1) blocks = 1;
  if (table)
    hipLaunchKernelGGL((cache_append_kernel<D, true, VARPOS>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)k_cache,
                       (uint16_t*)v_cache, (uint16_t*)k16,
                       static_cast<uint8_t*>(k16) + prefill_kexp_offset(B, Hkv, pos0 + Sq, D), n_bh, Sq,
                       S_max, pos0, conv_first, reinterpret_cast<const float2*>(table), pos0_dev, Hkv, window);
  else
    hipLaunchKernelGGL((cache_append_kernel<D, false, VARPOS>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)k_cache,
                       (uint16_t*)v_cache, (uint16_t*)nullptr, (uint8_t*)nullptr, n_bh, Sq, S_max, pos0, pos0,
                       (const float2*)nullptr, pos0_dev, Hkv, window);
  return hipGetLastError();
}

// VARPOS: chunks at per-sequence positions, as in cache_append_kernel: the grid covers rows
// [0, pos0 + Sq) of every (batch, KV head) (pos0: the largest start allowed, and the row count
// of the workspace copies), and sequence b, whose chunk starts at p = pos0_dev[b], writes its
// rows from its own conv_first (the tile of p - window; zeros before p - window) to p + Sq.  A
// sequence whose p lies outside [0, pos0] is left untouched.
template <int D, bool ROPE, bool VARPOS>
__global__ __launch_bounds__(256) void cache_append_paged_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_pages,
    uint16_t* __restrict__ v_pages, const int32_t* __restrict__ block_table, int max_blocks, int bs_log2,
    int num_blocks, uint16_t* __restrict__ k_ws, uint8_t* __restrict__ kexp, uint16_t* __restrict__ v_ws, int B,
    int Hkv, int Sq, int pos0_in, int conv_first, int first_seen_in, const float2* __restrict__ table,
    const int32_t* __restrict__ pos0_dev, int window) {
  constexpr int NCH = D / 8;  // 16-byte chunks per row
  const int Sk = pos0_in + Sq;  // rows per (batch, KV head) of the workspace copies
  const int first = VARPOS ? 0 : conv_first;
  const int nrows = Sk - first;
  const int64_t n = (int64_t)B * Hkv * nrows * NCH;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int cc = (int)(idx % NCH);
    const int64_t rr = idx / NCH;
    const int s = first + (int)(rr % nrows);
    const int64_t bh = rr / nrows;
    const int b = (int)(bh / Hkv), hkv = (int)(bh % Hkv);
    const int64_t wrow = (bh * Sk + s) * D + cc * 8;  // element offset in the workspace copies
    int pos0 = pos0_in, first_seen = first_seen_in;
    if constexpr (VARPOS) {
      // the NCH lanes of a row share s and b, so they skip together (to_f16_row needs all of them)
      pos0 = pos0_dev[b];
      if (pos0 < 0 || pos0 > pos0_in) continue;
      first_seen = window >= pos0 ? 0 : pos0 - window;
      if (s < (first_seen / 64) * 64 || s >= pos0 + Sq) continue;
    }
    // checked build, site 1: the row in the workspace copies, and its table entry
    if (!ATTN_IN(b < B && s >= 0 && s < Sk && (s >> bs_log2) < max_blocks, 1)) continue;
    if (s < first_seen) {
      // before every query's window (in the first tile the attention reads, masked there): never
      // read, so its block may have been released; zeros keep the masked products finite
      *reinterpret_cast<u32x4*>(k_ws + wrow) = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(v_ws + wrow) = u32x4{0, 0, 0, 0};
      if (ROPE && cc == 0) kexp[bh * Sk + s] = 0;
      continue;
    }
    int blk = block_table[(int64_t)b * max_blocks + (s >> bs_log2)];
    blk = min(max(blk, 0), num_blocks - 1);
    const int64_t prow = ((((int64_t)blk * Hkv + hkv) << bs_log2) + (s & ((1 << bs_log2) - 1))) * D + cc * 8;
    // checked build, site 2: the slot in the pool
    if (!ATTN_IN(prow + 8 <= ((int64_t)num_blocks * Hkv << bs_log2) * D, 2)) continue;
    if (s < pos0) {
      // earlier token: its stored key (to fp16 with RoPE) and value, gathered
      const u32x4 w = *reinterpret_cast<const u32x4*>(k_pages + prow);
      u32x4 h = w;
      if constexpr (ROPE) {
        const int e = to_f16_row<NCH>(w, h);
        if (cc == 0) kexp[bh * Sk + s] = (uint8_t)e;
      }
      *reinterpret_cast<u32x4*>(k_ws + wrow) = h;
      *reinterpret_cast<u32x4*>(v_ws + wrow) = *reinterpret_cast<const u32x4*>(v_pages + prow);
      continue;
    }
    const int64_t nrow = (bh * Sq + (s - pos0)) * D + cc * 8;  // element offset in the chunk
    const u32x4 kw = *reinterpret_cast<const u32x4*>(k_new + nrow);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(v_new + nrow);
    if constexpr (ROPE) {
      const u32x4 kb = rope_chunk_bf16<D>(kw, table, s, cc);
      u32x4 kh;
      const int e = to_f16_row<NCH>(kb, kh);
      if (cc == 0) kexp[bh * Sk + s] = (uint8_t)e;
      *reinterpret_cast<u32x4*>(k_pages + prow) = kb;
      *reinterpret_cast<u32x4*>(k_ws + wrow) = kh;
    } else {
      *reinterpret_cast<u32x4*>(k_pages + prow) = kw;
      *reinterpret_cast<u32x4*>(k_ws + wrow) = kw;
    }
    *reinterpret_cast<u32x4*>(v_pages + prow) = vw;
    *reinterpret_cast<u32x4*>(v_ws + wrow) = vw;
  }
}

template <int D, bool VARPOS>
hipError_t append_paged_go(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                           const int32_t* block_table, int max_blocks, int bs_log2, int num_blocks, void* k_ws,
                           void* v_ws, int B, int Hkv, int Sq, int pos0, int conv_first, int first_seen,
                           const float* table, const int32_t* pos0_dev, int window, hipStream_t st) {
  const int64_t n = (int64_t)B * Hkv * (pos0 + Sq - (VARPOS ? 0 : conv_first)) * (D / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 workgroups per CU
  if (blocks < 1) blocks = 1;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, (uint16_t*)k_pages, (uint16_t*)v_pages, block_table, max_blocks,
                       bs_log2, num_blocks, (uint16_t*)k_ws,
                       static_cast<uint8_t*>(k_ws) + prefill_kexp_offset(B, Hkv, pos0 + Sq, D), (uint16_t*)v_ws,
                       B, Hkv, Sq, pos0, conv_first, first_seen, reinterpret_cast<const float2*>(table), pos0_dev,
                       window);
    return hipGetLastError();
  };
  return table ? go(cache_append_paged_kernel<D, true, VARPOS>) : go(cache_append_paged_kernel<D, false, VARPOS>);
}

// Append only (the step before attn_decode in a serving loop): Sq new rows of every (batch, KV
// head) at per-sequence positions, sequence b's rows p .. p+Sq-1 with p = pos[b]; keys rotated in
// fp32 at their positions and rounded to bf16, values copied.  Into the contiguous cache
// [B*Hkv, S_max, D] or, PAGED, into the pool [num_blocks, Hkv, 1 << bs_log2, D] through the block
// table.  A sequence with p outside [0, s_cap - Sq] (s_cap: the rows the cache and, with RoPE, the
// table cover) is not written.
template <int D, bool ROPE, bool PAGED>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_dst,
    uint16_t* __restrict__ v_dst, const int32_t* __restrict__ pos, int64_t n_bh, int Hkv, int Sq, int S_max,
    int s_cap, const int32_t* __restrict__ block_table, int max_blocks, int bs_log2, int num_blocks,
    const float2* __restrict__ table) {
  constexpr int NCH = D / 8;  // 16-byte chunks per row
  const int64_t n = n_bh * Sq * NCH;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int cc = (int)(idx % NCH);
    const int64_t rr = idx / NCH;
    const int i = (int)(rr % Sq);
    const int64_t bh = rr / Sq;
    const int b = (int)(bh / Hkv), hkv = (int)(bh % Hkv);
    const int p = pos[b];
    if (p < 0 || p > s_cap - Sq) continue;
    const int s = p + i;
    int64_t drow;  // element offset of the row's chunk in the cache or pool
    if constexpr (PAGED) {
      // checked build, site 3: the table entry, then the slot in the pool
      if (!ATTN_IN((s >> bs_log2) < max_blocks, 3)) continue;
      int blk = block_table[(int64_t)b * max_blocks + (s >> bs_log2)];
      blk = min(max(blk, 0), num_blocks - 1);
      drow = ((((int64_t)blk * Hkv + hkv) << bs_log2) + (s & ((1 << bs_log2) - 1))) * D + cc * 8;
      if (!ATTN_IN(drow + 8 <= ((int64_t)num_blocks * Hkv << bs_log2) * D, 3)) continue;
    } else {
      drow = (bh * S_max + s) * D + cc * 8;
      // checked build, site 4: the row in the cache
      if (!ATTN_IN(s < S_max, 4)) continue;
    }
    const int64_t nrow = (bh * Sq + i) * D + cc * 8;  // element offset in the new rows
    const u32x4 kw = *reinterpret_cast<const u32x4*>(k_new + nrow);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(v_new + nrow);
    *reinterpret_cast<u32x4*>(k_dst + drow) = ROPE ? rope_chunk_bf16<D>(kw, table, s, cc) : kw;
    *reinterpret_cast<u32x4*>(v_dst + drow) = vw;
  }
}

template <int D>
hipError_t kv_append_go(const void* k_new, const void* v_new, void* k_dst, void* v_dst, const int32_t* pos, int B,
                        int Hkv, int Sq, int S_max, int s_cap, const int32_t* block_table, int max_blocks,
                        int bs_log2, int num_blocks, const float* table, hipStream_t st) {
  const int64_t n_bh = (int64_t)B * Hkv;
  int64_t blocks = (n_bh * Sq * (D / 8) + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 workgroups per CU
  if (blocks < 1) blocks = 1;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, (uint16_t*)k_dst, (uint16_t*)v_dst, pos, n_bh, Hkv, Sq, S_max, s_cap,
                       block_table, max_blocks, bs_log2, num_blocks, reinterpret_cast<const float2*>(table));
    return hipGetLastError();
  };
  if (block_table)
    return table ? go(kv_append_kernel<D, true, true>) : go(kv_append_kernel<D, false, true>);
  return table ? go(kv_append_kernel<D, true, false>) : go(kv_append_kernel<D, false, false>);
}

}  // namespace

ATTN_CHECK_READER(checked_word_cache)

hipError_t launch_cache_append_paged(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                                     const int32_t* block_table, int max_blocks, int bs_log2, int num_blocks,
                                     void* k_ws, void* v_ws, int B, int Hkv, int Sq, int D, int pos0,
                                     int conv_first, int first_seen, const float* table, hipStream_t st) {
  return D == 64 ? append_paged_go<64, false>(k_new, v_new, k_pages, v_pages, block_table, max_blocks, bs_log2,
                                              num_blocks, k_ws, v_ws, B, Hkv, Sq, pos0, conv_first, first_seen,
                                              table, nullptr, 0, st)
                 : append_paged_go<128, false>(k_new, v_new, k_pages, v_pages, block_table, max_blocks, bs_log2,
                                               num_blocks, k_ws, v_ws, B, Hkv, Sq, pos0, conv_first, first_seen,
                                               table, nullptr, 0, st);
}

hipError_t launch_cache_append_paged_varpos(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                                            const int32_t* block_table, int max_blocks, int bs_log2,
                                            int num_blocks, void* k_ws, void* v_ws, int B, int Hkv, int Sq, int D,
                                            int pos0_max, const int32_t* pos0_dev, int window, const float* table,
                                            hipStream_t st) {
  return D == 64 ? append_paged_go<64, true>(k_new, v_new, k_pages, v_pages, block_table, max_blocks, bs_log2,
                                             num_blocks, k_ws, v_ws, B, Hkv, Sq, pos0_max, 0, 0, table, pos0_dev,
                                             window, st)
                 : append_paged_go<128, true>(k_new, v_new, k_pages, v_pages, block_table, max_blocks, bs_log2,
                                              num_blocks, k_ws, v_ws, B, Hkv, Sq, pos0_max, 0, 0, table, pos0_dev,
                                              window, st);
}

hipError_t launch_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               void* k16, int B, int Hkv, int Sq, int S_max, int D, int pos0,
                               int conv_first, const float* table, hipStream_t st) {
  return D == 64 ? append_go<64, false>(k_new, v_new, k_cache, v_cache, k16, B, Hkv, Sq, S_max, pos0, conv_first,
                                        table, nullptr, 0, st)
                 : append_go<128, false>(k_new, v_new, k_cache, v_cache, k16, B, Hkv, Sq, S_max, pos0, conv_first,
                                         table, nullptr, 0, st);
}

hipError_t launch_cache_append_varpos(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                      void* k16, int B, int Hkv, int Sq, int S_max, int D, int pos0_max,
                                      const int32_t* pos0_dev, int window, const float* table, hipStream_t st) {
  return D == 64 ? append_go<64, true>(k_new, v_new, k_cache, v_cache, k16, B, Hkv, Sq, S_max, pos0_max, 0,
                                       table, pos0_dev, window, st)
                 : append_go<128, true>(k_new, v_new, k_cache, v_cache, k16, B, Hkv, Sq, S_max, pos0_max, 0,
                                        table, pos0_dev, window, st);
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_dst, void* v_dst, const int32_t* pos,
                            int B, int Hkv, int Sq, int D, int S_max, int s_cap, const int32_t* block_table,
                            int max_blocks, int bs_log2, int num_blocks, const float* table, hipStream_t st) {
  return D == 64 ? kv_append_go<64>(k_new, v_new, k_dst, v_dst, pos, B, Hkv, Sq, S_max, s_cap, block_table,
                                    max_blocks, bs_log2, num_blocks, table, st)
                 : kv_append_go<128>(k_new, v_new, k_dst, v_dst, pos, B, Hkv, Sq, S_max, s_cap, block_table,
                                     max_blocks, bs_log2, num_blocks, table, st);
}

}  // namespace attn
