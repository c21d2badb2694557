// float32 prefill: tiled exact attention with an online softmax, all arithmetic in fp32.
//
// This is the high-precision path (fp32 in, fp32 out): scaled dot-product attention of
// "Transformer Architecture & Self-Attention Mechanics" (devthesis.com) section 1, causal mask of
// the "Multi-Head Attention & Rotary Position Embeddings (RoPE)" listing (learnllm.online), RoPE
// of devthesis section 3 applied to Q and K as their tiles are loaded, and the tiling with a
// running max and sum of "Building Self-Attention and Transformer Engines" (codingpancake.com)
// section 4.1.  An optional sliding window (same page, section 6.4) limits each row to the
// `window` keys before it.
//
// One wave (64 lanes) owns 32 query rows; lanes l and l+32 hold the two halves of row l's head
// dimension, so the q and o vectors of a row live in registers and a dot product needs one
// cross-half exchange.  K (rotated on load) and V tiles of 32 keys are staged in LDS and read
// as broadcasts.
#include "common.h"

namespace attn {

namespace {

constexpr int kRows = 32;  // query rows per wave / workgroup
constexpr int kKeys = 32;  // keys per tile

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int S, int causal, int window,
    int pos0, const float2* __restrict__ table) {
  constexpr int H = D / 2;  // elements per lane
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];

  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int r = lane & 31;
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (Hq / Hkv);
  const int row = qb * kRows + r;
  const int row_c = row < S ? row : S - 1;
  // checked build, site 0: the workgroup's head, KV head and query block
  if (!ATTN_IN(h < Hq && kvh < Hkv && qb * kRows < S && Hq % Hkv == 0, 0)) return;

  const float* qrow = q + (((int64_t)b * Hq + h) * S + row_c) * D + half * H;
  float qv[H];
#pragma unroll
  for (int d = 0; d < H; ++d) qv[d] = qrow[d];
  if (table) {
    const float2* t = table + (int64_t)(pos0 + row_c) * (D / 2) + half * (H / 2);
#pragma unroll
    for (int p = 0; p < H / 2; ++p) {
      const float2 cs = t[p];
      const float x0 = qv[2 * p], x1 = qv[2 * p + 1];
      qv[2 * p] = x0 * cs.x - x1 * cs.y;
      qv[2 * p + 1] = x0 * cs.y + x1 * cs.x;
    }
  }
  const float scale = 1.0f / sqrtf((float)D);

  float acc[H];
#pragma unroll
  for (int d = 0; d < H; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const float* kbase = k + ((int64_t)b * Hkv + kvh) * S * D;
  const float* vbase = v + ((int64_t)b * Hkv + kvh) * S * D;
  const int last_row = min(qb * kRows + kRows, S) - 1;
  const int key_end = causal ? last_row + 1 : S;
  // visible keys of this row: [lo, hi] (causal: hi = row; sliding window: lo = row - window)
  const int hi = causal ? row : S - 1;
  const int lo = causal ? max(row - window, 0) : 0;
  const int key_begin = causal ? (max(0, qb * kRows - window) / kKeys) * kKeys : 0;

  for (int k0 = key_begin; k0 < key_end; k0 += kKeys) {
    __syncthreads();
    // Stage 32 keys: each lane moves pairs (2 floats) at a time, rotating K.
    for (int e = lane; e < kKeys * D / 2; e += 64) {
      const int kr = e / (D / 2);
      const int p = e - kr * (D / 2);
      const int key = k0 + kr;
      float2 kk = make_float2(0.f, 0.f), vv = make_float2(0.f, 0.f);
      if (key < S) {
        kk = *reinterpret_cast<const float2*>(kbase + (int64_t)key * D + 2 * p);
        vv = *reinterpret_cast<const float2*>(vbase + (int64_t)key * D + 2 * p);
        if (table) {
          const float2 cs = table[(int64_t)(pos0 + key) * (D / 2) + p];
          kk = make_float2(kk.x * cs.x - kk.y * cs.y, kk.x * cs.y + kk.y * cs.x);
        }
      }
      ks[kr][2 * p] = kk.x;
      ks[kr][2 * p + 1] = kk.y;
      vs[kr][2 * p] = vv.x;
      vs[kr][2 * p + 1] = vv.y;
    }
    __syncthreads();

    float s[kKeys];
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < H; ++d) part = fmaf(qv[d], ks[j][half * H + d], part);
      const float sj = (part + swap_halves(part)) * scale;
      const int key = k0 + j;
      s[j] = (key >= lo && key <= hi && key < S) ? sj : -INFINITY;
    }
    float m_tile = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) m_tile = fmaxf(m_tile, s[j]);
    const float m_new = fmaxf(m_run, m_tile);
    if (m_new == -INFINITY) continue;  // nothing visible yet for this row
    const float alpha = expf(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < H; ++d) acc[d] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = expf(s[j] - m_run);
      l_run += p;
#pragma unroll
      for (int d = 0; d < H; ++d) acc[d] = fmaf(p, vs[j][half * H + d], acc[d]);
    }
  }

  if (row < S) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* orow = o + (((int64_t)b * Hq + h) * S + row) * D + half * H;
#pragma unroll
    for (int d = 0; d < H; ++d) orow[d] = acc[d] * inv;
    if (lse && half == 0)
      lse[((int64_t)b * Hq + h) * S + row] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
  }
}

}  // namespace

ATTN_CHECK_READER(checked_word_prefill_f32)

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st) {
  dim3 grid((a.S + kRows - 1) / kRows, a.Hq, a.B);
  const float2* tab = reinterpret_cast<const float2*>(a.table);
  if (a.D == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(64), 0, st, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.Hq, a.Hkv, a.S,
                       (int)a.causal, a.window, a.pos0, tab);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(64), 0, st, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.Hq, a.Hkv, a.S,
                       (int)a.causal, a.window, a.pos0, tab);
  return hipGetLastError();
}

}  // namespace attn
