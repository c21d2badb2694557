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
// rope_apply is HBM-bound: it reads and writes every element once.  Each lane moves 16 bytes of x
// per head for bf16 (4 pairs) or fp32 (2 pairs), so loads and stores are dwordx4 and coalesced
// along D, and it reuses one load of its table entries for 4 heads.
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

// One row segment of 2*PPT elements of x at element offset e, widened to fp32.
template <bool BF16, int PPT>
__device__ __forceinline__ void rope_load(const void* x, int64_t e, float (&v)[2 * PPT]) {
  if constexpr (BF16) {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(x) + e;
    if constexpr (PPT == 4) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
#pragma unroll
      for (int j = 0; j < 4; ++j) { v[2 * j] = bf16lo(w[j]); v[2 * j + 1] = bf16hi(w[j]); }
    } else {
#pragma unroll
      for (int j = 0; j < 2 * PPT; ++j) v[j] = __uint_as_float((uint32_t)src[j] << 16);
    }
  } else {
    const float* src = reinterpret_cast<const float*>(x) + e;
    if constexpr (PPT == 2) {
      const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = w[j];
    } else {
#pragma unroll
      for (int j = 0; j < 2 * PPT; ++j) v[j] = src[j];
    }
  }
}

// Rotate the PPT pairs of v by the (cos, sin) entries cs and store them at element offset e:
// x0' = x0 c - x1 s, x1' = x0 s + x1 c, each as one fused multiply-add on a rounded product.
template <bool BF16, int PPT>
__device__ __forceinline__ void rope_rotate_store(void* out, int64_t e, const float (&v)[2 * PPT],
                                                  const float (&cs)[2 * PPT]) {
  float r[2 * PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const float x0 = v[2 * j], x1 = v[2 * j + 1], c = cs[2 * j], sn = cs[2 * j + 1];
    r[2 * j] = fmaf(x0, c, -(x1 * sn));
    r[2 * j + 1] = fmaf(x1, c, x0 * sn);
  }
  if constexpr (BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(out) + e;
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
    float* dst = reinterpret_cast<float*>(out) + e;
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

// PPT pairs per lane; each lane rotates the same pairs at one position s in HPT consecutive
// (batch, head) row blocks, so its table entries are loaded once for all of them, and for a full
// group the HPT loads of x are issued back to back.  x is [bh_count][S][D]; row (bh, s) sits at
// position pos0 + s.  x is read once, so its loads are nontemporal (in place, each element is
// read and then written by the same lane).
template <bool BF16, int PPT, int HPT>
__global__ __launch_bounds__(256) void rope_apply_kernel(const void* x, void* out, int64_t bh_count,
                                                         int S, int D, int pos0,
                                                         const float2* __restrict__ table) {
  const int half = D / 2;
  const int lanes_per_row = half / PPT;
  const int64_t n_groups = (bh_count + HPT - 1) / HPT;
  const int64_t per_group = (int64_t)S * lanes_per_row;
  const int64_t n = n_groups * per_group;
  const int64_t bh_stride = (int64_t)S * D;  // elements between the same (s, pair) of two row blocks
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t group = idx / per_group;
    const int64_t rem = idx - group * per_group;
    const int s = (int)(rem / lanes_per_row);
    const int p0 = (int)(rem - (int64_t)s * lanes_per_row) * PPT;  // first pair of this lane
    // checked build, site 0: the last element of the last row block this lane touches
    if (!ATTN_IN(s < S && p0 + PPT <= half &&
                     ((group * HPT + min<int64_t>(HPT, bh_count - group * HPT) - 1) * S + s) * D + 2 * (p0 + PPT) <=
                         bh_count * bh_stride,
                 0))
      continue;
    const float2* tr = table + (int64_t)(pos0 + s) * half + p0;
    float cs[2 * PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) { const float2 t = tr[j]; cs[2 * j] = t.x; cs[2 * j + 1] = t.y; }
    const int64_t bh0 = group * HPT;
    const int64_t base = (bh0 * S + s) * D + 2 * p0;
    if (bh_count - bh0 >= HPT) {
      float v[HPT][2 * PPT];
#pragma unroll
      for (int h = 0; h < HPT; ++h) rope_load<BF16, PPT>(x, base + h * bh_stride, v[h]);
#pragma unroll
      for (int h = 0; h < HPT; ++h) rope_rotate_store<BF16, PPT>(out, base + h * bh_stride, v[h], cs);
    } else {
      const int nh = (int)(bh_count - bh0);
      for (int h = 0; h < nh; ++h) {
        float v[2 * PPT];
        rope_load<BF16, PPT>(x, base + h * bh_stride, v);
        rope_rotate_store<BF16, PPT>(out, base + h * bh_stride, v, cs);
      }
    }
  }
}

template <bool BF16, int PPT>
static hipError_t rope_apply_go(const void* x, void* out, int64_t rows, int S, int D, int pos0,
                                const float* table, hipStream_t st) {
  constexpr int HPT = 4;
  const int64_t bh_count = rows / S;
  const int64_t n = (bh_count + HPT - 1) / HPT * S * (D / 2 / PPT);
  const int threads = 256;
  int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 16384) blocks = 16384;  // grid-stride beyond 64 blocks per CU
  hipLaunchKernelGGL((rope_apply_kernel<BF16, PPT, HPT>), dim3((unsigned)blocks), dim3(threads), 0, st,
                     x, out, bh_count, S, D, pos0, reinterpret_cast<const float2*>(table));
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
// table) and store it as fp16, the operand format of the Q.K^T product of the bf16 prefill, with
// the row's power-of-two exponent (f16_row_exponent: rows reaching 2^15 are stored scaled down,
// their exponent byte in kexp [bh_count, S]).  K is not read again, so its loads are nontemporal
// and leave the caches to the fp16 copy and V (a whole MHA step at 2k tokens +1 to +5%).
template <int D, int HPT>
__global__ __launch_bounds__(256) void rope_k_f16_kernel(const uint16_t* __restrict__ k,
                                                         uint16_t* __restrict__ out, uint8_t* __restrict__ kexp,
                                                         int64_t bh_count, int S, int pos0,
                                                         const float2* __restrict__ table) {
  // Each lane rotates 4 pairs at one position in HPT consecutive (batch, head) row blocks: one
  // load of its table entries serves all of them, and a full group's loads issue back to back.
  // The NCH lanes of one row are consecutive (aligned), so a row's maximum is a group reduction.
  constexpr int NCH = D / 8;
  const int64_t n_groups = (bh_count + HPT - 1) / HPT;
  const int64_t per_group = (int64_t)S * NCH;
  const int64_t n = n_groups * per_group;
  const int64_t bh_stride = (int64_t)S * D;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t group = idx / per_group;
    const int64_t rem = idx - group * per_group;
    const int s = (int)(rem / NCH);
    const int cc = (int)(rem - (int64_t)s * NCH);
    const f32x4* tp = reinterpret_cast<const f32x4*>(table + (int64_t)(pos0 + s) * (D / 2) + cc * 4);
    const f32x4 c01 = tp[0], c23 = tp[1];
    const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
    const int64_t bh0 = group * HPT;
    const int64_t base = (bh0 * S + s) * D + cc * 8;
    const int nh = bh_count - bh0 < HPT ? (int)(bh_count - bh0) : HPT;
    // checked build, site 1: the last key element and exponent byte of this lane's row blocks
    if (!ATTN_IN(s < S && cc < NCH && base + (nh - 1) * bh_stride + 8 <= bh_count * bh_stride &&
                     (bh0 + nh - 1) * S + s < bh_count * S,
                 1))
      continue;
    // rotate, then scale the row by its exponent and store it as fp16
    auto rotate_store = [&](const u32x4 w, int hh) {
      float r[8];
      float mx = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = bf16lo(w[p]), x1 = bf16hi(w[p]);
        const float c = cs[2 * p], sn = cs[2 * p + 1];
        r[2 * p] = fmaf(x0, c, -(x1 * sn));
        r[2 * p + 1] = fmaf(x1, c, x0 * sn);
        mx = fmaxf(mx, fmaxf(fabsf(r[2 * p]), fabsf(r[2 * p + 1])));
      }
      const int e = f16_row_exponent(group_max<NCH>(mx));
      u32x4 hw;
#pragma unroll
      for (int p = 0; p < 4; ++p) hw[p] = pack_f16(ldexpf(r[2 * p], -e), ldexpf(r[2 * p + 1], -e));
      *reinterpret_cast<u32x4*>(out + base + hh * bh_stride) = hw;
      if (cc == 0) kexp[(bh0 + hh) * S + s] = (uint8_t)e;
    };
    if (nh == HPT) {
      u32x4 w[HPT];
#pragma unroll
      for (int h = 0; h < HPT; ++h)
        w[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + base + h * bh_stride));
#pragma unroll
      for (int h = 0; h < HPT; ++h) rotate_store(w[h], h);
    } else {
      for (int h = 0; h < nh; ++h)
        rotate_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + base + h * bh_stride)), h);
    }
  }
}

template <int D>
static hipError_t rotate_keys(const void* k, void* k_rot, int64_t rows, int S, int pos0, const float* table,
                       hipStream_t st) {
  constexpr int HPT = 4;
  const int64_t bh_count = rows / S;
  int64_t blocks = ((bh_count + HPT - 1) / HPT * S * (D / 8) + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  uint8_t* kexp = static_cast<uint8_t*>(k_rot) + rows * D * 2;
  hipLaunchKernelGGL((rope_k_f16_kernel<D, HPT>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint16_t*)k, (uint16_t*)k_rot, kexp, bh_count, S, pos0,
                     reinterpret_cast<const float2*>(table));
  return hipGetLastError();
}

ATTN_CHECK_READER(checked_word_rope)

hipError_t launch_rotate_keys_f16(const void* k, void* k_rot, int B, int Hkv, int S, int D, int pos0,
                                  const float* table, hipStream_t st) {
  const int64_t rows = (int64_t)B * Hkv * S;
  return D == 64 ? rotate_keys<64>(k, k_rot, rows, S, pos0, table, st)
                 : rotate_keys<128>(k, k_rot, rows, S, pos0, table, st);
}

}  // namespace attn
