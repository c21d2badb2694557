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
//    the new rows from the very bf16 values just stored (bf16 -> fp16 is exact for
//    6.1e-5 <= |x| <= 65504; smaller magnitudes round to fp16's subnormal grid, 2^-24).
//
// Paged cache (cache_append_paged_kernel): the pool [num_blocks, Hkv, bs, D] and block table of
// codingpancake.com "Building Self-Attention and Transformer Engines", section 6.2; token t of
// sequence b sits in block block_table[b][t / bs], slot t % bs.  The new rows go into their
// blocks as above, and every row the attention can read, [conv_first, pos0+Sq), is also gathered
// into contiguous workspace copies: the keys (fp16 with RoPE, bf16 without) and the values
// (bf16), which the attention kernel then streams as it streams a contiguous cache.  Rows before
// first_seen (the first query's window start; no query sees them) are written as zeros instead
// of being read, so blocks wholly before it, and their table entries, are never touched.
#include "common.h"

namespace attn {

namespace {

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void cache_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, uint16_t* __restrict__ k16,
    int64_t n_bh, int Sq, int S_max, int pos0, int conv_first, const float2* __restrict__ table) {
  constexpr int NCH = D / 8;  // 16-byte chunks per row
  // rows handled per (batch, KV head): [first, pos0 + Sq); with RoPE the earlier rows from
  // conv_first on (those a sliding window can still see) are converted to fp16
  const int first = ROPE ? conv_first : pos0;
  const int Sk = pos0 + Sq;
  const int nrows = Sk - first;
  const int64_t n = n_bh * nrows * NCH;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int cc = (int)(idx % NCH);
    const int64_t rr = idx / NCH;
    const int s = first + (int)(rr % nrows);
    const int64_t bh = rr / nrows;
    const int64_t crow = (bh * S_max + s) * D + cc * 8;  // element offset in the cache
    if (s < pos0) {
      // earlier token (RoPE only): its stored bf16 key, converted to fp16
      const u32x4 w = *reinterpret_cast<const u32x4*>(k_cache + crow);
      u32x4 h;
#pragma unroll
      for (int t = 0; t < 4; ++t) h[t] = pack_f16(bf16lo(w[t]), bf16hi(w[t]));
      *reinterpret_cast<u32x4*>(k16 + (bh * Sk + s) * D + cc * 8) = h;
      continue;
    }
    const int64_t nrow = (bh * Sq + (s - pos0)) * D + cc * 8;  // element offset in the chunk
    const u32x4 kw = *reinterpret_cast<const u32x4*>(k_new + nrow);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(v_new + nrow);
    if constexpr (ROPE) {
      const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)s * (D / 2) + cc * 4);
      const f32x4 c01 = tp[0], c23 = tp[1];
      const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
      u32x4 kb, kh;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = bf16lo(kw[p]), x1 = bf16hi(kw[p]);
        const float c = cs[2 * p], sn = cs[2 * p + 1];
        kb[p] = pack_bf16(x0 * c - x1 * sn, x0 * sn + x1 * c);
        kh[p] = pack_f16(bf16lo(kb[p]), bf16hi(kb[p]));
      }
      *reinterpret_cast<u32x4*>(k_cache + crow) = kb;
      *reinterpret_cast<u32x4*>(k16 + (bh * Sk + s) * D + cc * 8) = kh;
    } else {
      *reinterpret_cast<u32x4*>(k_cache + crow) = kw;
    }
    *reinterpret_cast<u32x4*>(v_cache + crow) = vw;
  }
}

template <int D>
hipError_t append_go(const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* k16,
                     int B, int Hkv, int Sq, int S_max, int pos0, int conv_first, const float* table,
                     hipStream_t st) {
  const int64_t n_bh = (int64_t)B * Hkv;
  const int64_t rows = table ? (int64_t)(pos0 + Sq - conv_first) : (int64_t)Sq;
  const int64_t n = n_bh * rows * (D / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 workgroups per CU
  if (blocks < 1) blocks = 1;
  if (table)
    hipLaunchKernelGGL((cache_append_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)k_cache,
                       (uint16_t*)v_cache, (uint16_t*)k16, n_bh, Sq, S_max, pos0, conv_first,
                       reinterpret_cast<const float2*>(table));
  else
    hipLaunchKernelGGL((cache_append_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)k_cache,
                       (uint16_t*)v_cache, (uint16_t*)nullptr, n_bh, Sq, S_max, pos0, pos0,
                       (const float2*)nullptr);
  return hipGetLastError();
}

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void cache_append_paged_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_pages,
    uint16_t* __restrict__ v_pages, const int32_t* __restrict__ block_table, int max_blocks, int bs_log2,
    int num_blocks, uint16_t* __restrict__ k_ws, uint16_t* __restrict__ v_ws, int B, int Hkv, int Sq,
    int pos0, int conv_first, int first_seen, const float2* __restrict__ table) {
  constexpr int NCH = D / 8;  // 16-byte chunks per row
  const int Sk = pos0 + Sq;
  const int nrows = Sk - conv_first;
  const int64_t n = (int64_t)B * Hkv * nrows * NCH;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int cc = (int)(idx % NCH);
    const int64_t rr = idx / NCH;
    const int s = conv_first + (int)(rr % nrows);
    const int64_t bh = rr / nrows;
    const int b = (int)(bh / Hkv), hkv = (int)(bh % Hkv);
    const int64_t wrow = (bh * Sk + s) * D + cc * 8;  // element offset in the workspace copies
    if (s < first_seen) {
      // before every query's window (in the first tile the attention reads, masked there): never
      // read, so its block may have been released; zeros keep the masked products finite
      *reinterpret_cast<u32x4*>(k_ws + wrow) = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(v_ws + wrow) = u32x4{0, 0, 0, 0};
      continue;
    }
    int blk = block_table[(int64_t)b * max_blocks + (s >> bs_log2)];
    blk = min(max(blk, 0), num_blocks - 1);
    const int64_t prow = ((((int64_t)blk * Hkv + hkv) << bs_log2) + (s & ((1 << bs_log2) - 1))) * D + cc * 8;
    if (s < pos0) {
      // earlier token: its stored key (to fp16 with RoPE) and value, gathered
      const u32x4 w = *reinterpret_cast<const u32x4*>(k_pages + prow);
      u32x4 h = w;
      if constexpr (ROPE) {
#pragma unroll
        for (int t = 0; t < 4; ++t) h[t] = pack_f16(bf16lo(w[t]), bf16hi(w[t]));
      }
      *reinterpret_cast<u32x4*>(k_ws + wrow) = h;
      *reinterpret_cast<u32x4*>(v_ws + wrow) = *reinterpret_cast<const u32x4*>(v_pages + prow);
      continue;
    }
    const int64_t nrow = (bh * Sq + (s - pos0)) * D + cc * 8;  // element offset in the chunk
    const u32x4 kw = *reinterpret_cast<const u32x4*>(k_new + nrow);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(v_new + nrow);
    if constexpr (ROPE) {
      const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)s * (D / 2) + cc * 4);
      const f32x4 c01 = tp[0], c23 = tp[1];
      const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
      u32x4 kb, kh;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = bf16lo(kw[p]), x1 = bf16hi(kw[p]);
        const float c = cs[2 * p], sn = cs[2 * p + 1];
        kb[p] = pack_bf16(x0 * c - x1 * sn, x0 * sn + x1 * c);
        kh[p] = pack_f16(bf16lo(kb[p]), bf16hi(kb[p]));
      }
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

template <int D>
hipError_t append_paged_go(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                           const int32_t* block_table, int max_blocks, int bs_log2, int num_blocks, void* k_ws,
                           void* v_ws, int B, int Hkv, int Sq, int pos0, int conv_first, int first_seen,
                           const float* table, hipStream_t st) {
  const int64_t n = (int64_t)B * Hkv * (pos0 + Sq - conv_first) * (D / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 workgroups per CU
  if (blocks < 1) blocks = 1;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, (uint16_t*)k_pages, (uint16_t*)v_pages, block_table, max_blocks,
                       bs_log2, num_blocks, (uint16_t*)k_ws, (uint16_t*)v_ws, B, Hkv, Sq, pos0, conv_first,
                       first_seen, reinterpret_cast<const float2*>(table));
    return hipGetLastError();
  };
  return table ? go(cache_append_paged_kernel<D, true>) : go(cache_append_paged_kernel<D, false>);
}

}  // namespace

hipError_t launch_cache_append_paged(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                                     const int32_t* block_table, int max_blocks, int bs_log2, int num_blocks,
                                     void* k_ws, void* v_ws, int B, int Hkv, int Sq, int D, int pos0,
                                     int conv_first, int first_seen, const float* table, hipStream_t st) {
  return D == 64 ? append_paged_go<64>(k_new, v_new, k_pages, v_pages, block_table, max_blocks, bs_log2,
                                       num_blocks, k_ws, v_ws, B, Hkv, Sq, pos0, conv_first, first_seen, table, st)
                 : append_paged_go<128>(k_new, v_new, k_pages, v_pages, block_table, max_blocks, bs_log2,
                                        num_blocks, k_ws, v_ws, B, Hkv, Sq, pos0, conv_first, first_seen, table,
                                        st);
}

hipError_t launch_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               void* k16, int B, int Hkv, int Sq, int S_max, int D, int pos0,
                               int conv_first, const float* table, hipStream_t st) {
  return D == 64 ? append_go<64>(k_new, v_new, k_cache, v_cache, k16, B, Hkv, Sq, S_max, pos0, conv_first,
                                 table, st)
                 : append_go<128>(k_new, v_new, k_cache, v_cache, k16, B, Hkv, Sq, S_max, pos0, conv_first,
                                  table, st);
}

}  // namespace attn
