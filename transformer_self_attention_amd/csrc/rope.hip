// Rotary position embeddings: coefficient table, the stand-alone rotation kernel, and the key
// rotation pass of the bf16 prefill (rotated keys stored as fp16).
//
// The rotation follows "Transformer Architecture & Self-Attention Mechanics" (devthesis.com),
// section 3, "Rotary Position Embeddings (RoPE)": adjacent pairs (x[2i], x[2i+1]) of a head
// vector at position m are turned counter-clockwise by m * theta_i, theta_i = base^(-2i/D).
// The frequencies match the NumPy example of "Transformer Architecture: FlashAttention & RoPE"
// (academy.kwas.tech).
//
// Frequency scalings for contexts past the trained length (named on ninaddeshpande.com "Transformer
// internals", "Rotary positional embeddings (RoPE)", and devthesis Problem 3; formulas from their
// publications): position interpolation divides positions by the factor s; NTK-aware scaling
// raises the base to base * s^(D/(D-2)); YaRN interpolates each pair by its wavelength (ramp over
// r = original context / wavelength between beta_slow and beta_fast) and scales cos and sin by
// 0.1 ln(s) + 1.  Only the table changes: every kernel reads the rotation from it.
//
// rope_apply is HBM-bound: it reads and writes every element once (plus the table row, which
// stays in L2 across heads).  Each lane moves 16 bytes of x for bf16 (4 pairs) or fp32
// (2 pairs), so loads and stores are dwordx4 and coalesced along D.
#include "common.h"

namespace attn {

// table[m][i] = amp * (cos(a), sin(a)), a = m * theta_i (plain), with the scaling applied to m,
// theta_i and amp as above; every step in double precision, rounded once to float.
__global__ void rope_table_kernel(float2* __restrict__ table, int max_pos, int half, double base,
                                  RopeScalingArgs sc) {
  const int64_t n = (int64_t)max_pos * half;
  const double D = 2.0 * half;
  const double kPi = 3.14159265358979323846;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(idx / half);
    const int i = (int)(idx - (int64_t)m * half);
    double theta = pow(base, -2.0 * (double)i / D);
    double pos = (double)m, amp = 1.0;
    if (sc.kind == kRopePI) {
      pos = (double)m / sc.factor;
    } else if (sc.kind == kRopeNTK) {
      theta = pow(base * pow(sc.factor, D / (D - 2.0)), -2.0 * (double)i / D);
    } else if (sc.kind == kRopeYaRN) {
      const double r = sc.original_max_pos * theta / (2.0 * kPi);
      double g = (r - sc.beta_slow) / (sc.beta_fast - sc.beta_slow);
      g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
      theta = (1.0 - g) * theta / sc.factor + g * theta;
      amp = 0.1 * log(sc.factor) + 1.0;
    }
    const double ang = pos * theta;
    table[idx] = make_float2((float)(amp * cos(ang)), (float)(amp * sin(ang)));
  }
}

hipError_t launch_rope_table(float* table, int max_pos, int D, double base, const RopeScalingArgs& sc,
                             hipStream_t st) {
  const int half = D / 2;
  const int64_t n = (int64_t)max_pos * half;
  const int threads = 256;
  int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(threads), 0, st,
                     reinterpret_cast<float2*>(table), max_pos, half, base, sc);
  return hipGetLastError();
}

// PPT pairs per lane.  Rows are [rows_total = B*H*S][D]; row r sits at position pos0 + r % S.
template <bool BF16, int PPT>
__global__ void rope_apply_kernel(const void* x, void* out, int64_t rows,
                                  int S, int D, int pos0, const float2* __restrict__ table) {
  const int half = D / 2;
  const int lanes_per_row = half / PPT;
  const int64_t n = rows * lanes_per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / lanes_per_row;
    const int p0 = (int)(idx - row * lanes_per_row) * PPT;  // first pair of this lane
    const int pos = pos0 + (int)(row % S);
    const float2* tr = table + (int64_t)pos * half + p0;
    float v[2 * PPT];
    if constexpr (BF16) {
      const uint16_t* src = reinterpret_cast<const uint16_t*>(x) + row * D + 2 * p0;
      if constexpr (PPT == 4) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[2 * j] = bf16lo(w[j]); v[2 * j + 1] = bf16hi(w[j]); }
      } else {
#pragma unroll
        for (int j = 0; j < 2 * PPT; ++j) v[j] = __uint_as_float((uint32_t)src[j] << 16);
      }
    } else {
      const float* src = reinterpret_cast<const float*>(x) + row * D + 2 * p0;
      if constexpr (PPT == 2) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = w[j];
      } else {
#pragma unroll
        for (int j = 0; j < 2 * PPT; ++j) v[j] = src[j];
      }
    }
    float r[2 * PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const float2 cs = tr[j];
      r[2 * j] = v[2 * j] * cs.x - v[2 * j + 1] * cs.y;
      r[2 * j + 1] = v[2 * j] * cs.y + v[2 * j + 1] * cs.x;
    }
    if constexpr (BF16) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(out) + row * D + 2 * p0;
      if constexpr (PPT == 4) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack_bf16(r[2 * j], r[2 * j + 1]);
        *reinterpret_cast<u32x4*>(dst) = w;
      } else {
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
          const uint32_t w = pack_bf16(r[2 * j], r[2 * j + 1]);
          dst[2 * j] = (uint16_t)(w & 0xffffu);
          dst[2 * j + 1] = (uint16_t)(w >> 16);
        }
      }
    } else {
      float* dst = reinterpret_cast<float*>(out) + row * D + 2 * p0;
      if constexpr (PPT == 2) {
        f32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = r[j];
        *reinterpret_cast<f32x4*>(dst) = w;
      } else {
#pragma unroll
        for (int j = 0; j < 2 * PPT; ++j) dst[j] = r[j];
      }
    }
  }
}

template <bool BF16, int PPT>
static hipError_t rope_apply_go(const void* x, void* out, int64_t rows, int S, int D, int pos0,
                                const float* table, hipStream_t st) {
  const int64_t n = rows * (D / 2 / PPT);
  const int threads = 256;
  int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 blocks per CU
  hipLaunchKernelGGL((rope_apply_kernel<BF16, PPT>), dim3((unsigned)blocks), dim3(threads), 0, st,
                     x, out, rows, S, D, pos0, reinterpret_cast<const float2*>(table));
  return hipGetLastError();
}

hipError_t launch_rope_apply(const void* x, void* out, bool bf16, int64_t rows, int S, int D,
                             int pos0, const float* table, hipStream_t st) {
  const int half = D / 2;
  if (bf16) {
    if (half % 4 == 0) return rope_apply_go<true, 4>(x, out, rows, S, D, pos0, table, st);
    return rope_apply_go<true, 1>(x, out, rows, S, D, pos0, table, st);
  }
  if (half % 2 == 0) return rope_apply_go<false, 2>(x, out, rows, S, D, pos0, table, st);
  return rope_apply_go<false, 1>(x, out, rows, S, D, pos0, table, st);
}


// One pass over K: rotate every row at position pos0 + s (fp32 arithmetic, the same coefficient
// table) and store it as fp16, the operand format of the Q.K^T product of the bf16 prefill.  K is
// not read again, so its loads are nontemporal and leave the caches to the fp16 copy and V (a
// whole MHA step at 2k tokens +1 to +5%).
template <int D>
__global__ __launch_bounds__(256) void rope_k_f16_kernel(const uint16_t* __restrict__ k,
                                                         uint16_t* __restrict__ out, int64_t rows, int S,
                                                         int pos0, const float2* __restrict__ table) {
  constexpr int NCH = D / 8;
  const int64_t n = rows * NCH;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / NCH;
    const int cc = (int)(idx - r * NCH);
    const int pos = pos0 + (int)(r % S);
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + r * D + cc * 8));
    const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)pos * (D / 2) + cc * 4);
    const f32x4 c01 = tp[0], c23 = tp[1];
    const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
    u32x4 hw;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = bf16lo(w[p]), x1 = bf16hi(w[p]);
      const float c = cs[2 * p], s = cs[2 * p + 1];
      hw[p] = pack_f16(x0 * c - x1 * s, x0 * s + x1 * c);
    }
    *reinterpret_cast<u32x4*>(out + r * D + cc * 8) = hw;
  }
}

template <int D>
static hipError_t rotate_keys(const void* k, void* k_rot, int64_t rows, int S, int pos0, const float* table,
                       hipStream_t st) {
  int64_t blocks = (rows * (D / 8) + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(rope_k_f16_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint16_t*)k, (uint16_t*)k_rot, rows, S, pos0,
                     reinterpret_cast<const float2*>(table));
  return hipGetLastError();
}

hipError_t launch_rotate_keys_f16(const void* k, void* k_rot, int B, int Hkv, int S, int D, int pos0,
                                  const float* table, hipStream_t st) {
  const int64_t rows = (int64_t)B * Hkv * S;
  return D == 64 ? rotate_keys<64>(k, k_rot, rows, S, pos0, table, st)
                 : rotate_keys<128>(k, k_rot, rows, S, pos0, table, st);
}

}  // namespace attn
