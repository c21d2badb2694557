// Internal declarations shared by the HIP sources of libattn.so (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

// bfloat16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two packed bfloat16 (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Two floats -> two packed IEEE halves (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v;
  v[0] = (_Float16)a;
  v[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Value of lane (l xor 32) for every lane l, via v_permlane32_swap.
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const bool upper = (threadIdx.x & 32) != 0;
  return __uint_as_float(upper ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A value known to be the same in every lane, moved to a scalar register.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---- the checked build ----
// Built with ATTN_CHECKED defined, the kernels test the largest index each thread is about to use
// against the extents their own arguments give, at the point where that thread's index set is
// fixed.  A failed test sets bit `site` of this source file's check word and the thread skips the
// accesses it guards, so a bad index shows as a reported site instead of a memory fault; the
// words are read and cleared through attn_checked_sites().  Every test holds for a whole row (or
// a whole wave), so the lanes that share a row reduction stay together.  In the normal build
// ATTN_IN(cond, site) is the constant true and the tests compile away.
#ifdef ATTN_CHECKED
namespace {
__device__ unsigned int g_check_word;  // one per source file
}
__device__ __forceinline__ bool checked_in(bool ok, int site) {
  if (!ok) atomicOr(&g_check_word, 1u << site);
  return ok;
}
#define ATTN_IN(cond, site) (::attn::checked_in((cond), (site)))
// Host reader of this source file's word (read, then cleared), named `fn`.
#define ATTN_CHECK_READER(fn)                                                                      \
  unsigned int fn() {                                                                              \
    unsigned int w = 0, zero = 0;                                                                  \
    if (hipMemcpyFromSymbol(&w, HIP_SYMBOL(g_check_word), sizeof(w), 0, hipMemcpyDeviceToHost) != \
        hipSuccess)                                                                                \
      return ~0u;                                                                                  \
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_check_word), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) != \
        hipSuccess)                                                                                \
      return ~0u;                                                                                  \
    return w;                                                                                      \
  }
unsigned int checked_word_rope();
unsigned int checked_word_cache();
unsigned int checked_word_prefill_bf16();
unsigned int checked_word_prefill_f32();
unsigned int checked_word_decode();
unsigned int checked_word_decode_wide();
#else
#define ATTN_IN(cond, site) true
#define ATTN_CHECK_READER(fn)
#endif

// ---- fp16 operands with a power-of-two row exponent ----
// The Q.K^T products of the bf16 prefill take IEEE half operands (11 significant bits against
// bf16's 8), whose range ends at 65504.  A row whose largest magnitude reaches 2^15 is stored
// scaled by 2^-e, the smallest e >= 0 that brings it below 2^15 (so rounding to half cannot
// overflow), and e is kept beside it; scaling by a power of two is exact, and rows with e = 0 are
// stored exactly as before.  Non-finite rows keep e = 0.
__device__ __forceinline__ int f16_row_exponent(float max_abs) {
  const int eb = (int)((__float_as_uint(max_abs) >> 23) & 0xff);  // biased exponent
  if (eb == 255) return 0;
  const int u = eb - 127;  // max_abs in [2^u, 2^(u+1))
  return u > 14 ? u - 14 : 0;
}

// Maximum of x over each aligned group of N consecutive lanes (N = 8 or 16), in every lane of
// the group (DPP within rows of 16 lanes; all lanes of a group must be active).
template <int N>
__device__ __forceinline__ float group_max(float x) {
  static_assert(N == 8 || N == 16, "group size");
#define ATTN_DPP_MAX(v, ctrl) \
  fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, false)))
  x = ATTN_DPP_MAX(x, 0xb1);   // quad_perm [1, 0, 3, 2]
  x = ATTN_DPP_MAX(x, 0x4e);   // quad_perm [2, 3, 0, 1]
  x = ATTN_DPP_MAX(x, 0x141);  // row_half_mirror: lanes i and 7 - i of each 8
  if constexpr (N == 16) x = ATTN_DPP_MAX(x, 0x140);  // row_mirror: lanes i and 15 - i of each 16
#undef ATTN_DPP_MAX
  return x;
}

// ------------------------------------------------------------------------------------------
// Launchers (each returns hipGetLastError() of its launch).  Arguments were validated by the
// C-ABI layer; the launchers only size grids.
// ------------------------------------------------------------------------------------------
// RoPE frequency scaling of the coefficient table (kind: kRopePlain, kRopePI, kRopeNTK, kRopeYaRN).
enum { kRopePlain = 0, kRopePI = 1, kRopeNTK = 2, kRopeYaRN = 3 };
struct RopeScalingArgs {
  int kind;
  double factor;            // s >= 1
  double original_max_pos;  // YaRN: the trained context length
  double beta_fast, beta_slow;
};

hipError_t launch_rope_table(float* table, int max_pos, int D, double base, const RopeScalingArgs& sc,
                             hipStream_t st);

hipError_t launch_rope_apply(const void* x, void* out, bool bf16, int64_t rows, int S, int D,
                             int pos0, const float* table, hipStream_t st);

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  bool out_bf16;
  int B, Hq, Hkv, S, D;  // S: query rows per (batch, head)
  bool causal;
  int pos0;            // RoPE position of query row 0 (and of key row 0 when keys are rotated here)
  const float* table;  // nullptr: no RoPE
  void* workspace;     // bf16 path: room for the rotated fp16 keys, or nullptr (RoPE fused)
  // Keys: Sk rows per (batch, KV head), stored k_rows / v_rows rows apart (K / V); query row i
  // sees key j when j <= i + coff.  An ordinary prefill has Sk = k_rows = v_rows = S, coff = 0.
  int Sk, k_rows, v_rows, coff;
  // Sliding window: key j is visible to row i only if j >= i + coff - window (no window: 1 << 30).
  int window;
  // Chunks at per-sequence positions (chunked prefill only): sequence b's chunk starts at
  // pos0_dev[b] (device int32 [B]), which then replaces pos0 and coff, and Sk = pos0_dev[b] + S;
  // coff holds the largest start allowed.  nullptr: one position for the batch.
  const int32_t* pos0_dev = nullptr;
};

// Rotated keys as fp16 [B, Hkv, S, D], then one exponent byte per key row [B, Hkv, S] at byte
// offset prefill_kexp_offset(...) (the rows' scale, see f16_row_exponent).
size_t prefill_workspace_bytes(int B, int Hkv, int S, int D);
inline size_t prefill_kexp_offset(int B, int Hkv, int S, int D) { return (size_t)B * Hkv * S * D * 2; }
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st);
hipError_t launch_rotate_keys_f16(const void* k, void* k_rot, int B, int Hkv, int S, int D, int pos0,
                                  const float* table, hipStream_t st);
hipError_t launch_prefill_prerotated(const PrefillArgs& a, const void* k_rot, hipStream_t st);

// Chunked prefill against a KV cache (bf16): append the chunk's keys (rotated, rounded to bf16)
// and values to cache rows [pos0, pos0 + Sq); with RoPE also write key rows [conv_first,
// pos0 + Sq) as fp16 into k16 ([B*Hkv, pos0 + Sq, D]), the operand format of the Q.K^T product
// (rows before conv_first are never read: a sliding window no longer reaches them).
hipError_t launch_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               void* k16, int B, int Hkv, int Sq, int S_max, int D, int pos0,
                               int conv_first, const float* table, hipStream_t st);
// The same with per-sequence chunk starts pos0_dev[b] (device int32 [B], each in [0, pos0_max]):
// k16 holds pos0_max + Sq rows per (batch, KV head); window (kernel form, 1 << 30: none) sets
// each sequence's first fp16 row; a sequence whose start is out of range is not written.
hipError_t launch_cache_append_varpos(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                      void* k16, int B, int Hkv, int Sq, int S_max, int D, int pos0_max,
                                      const int32_t* pos0_dev, int window, const float* table, hipStream_t st);
// The same for a paged cache: pools [num_blocks, Hkv, 1 << bs_log2, D] and a block table
// [B, max_blocks].  The new rows go into their blocks; rows [conv_first, pos0 + Sq) are also
// gathered into k_ws (fp16 with RoPE, bf16 without) and v_ws (bf16), both [B*Hkv, pos0 + Sq, D]
// (rows before first_seen, which no query sees, as zeros without reading them).
hipError_t launch_cache_append_paged(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                                     const int32_t* block_table, int max_blocks, int bs_log2, int num_blocks,
                                     void* k_ws, void* v_ws, int B, int Hkv, int Sq, int D, int pos0,
                                     int conv_first, int first_seen, const float* table, hipStream_t st);
// The same with per-sequence chunk starts pos0_dev[b] in [0, pos0_max] (k_ws / v_ws hold
// pos0_max + Sq rows per (batch, KV head); window in kernel form sets each sequence's rows).
hipError_t launch_cache_append_paged_varpos(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                                            const int32_t* block_table, int max_blocks, int bs_log2,
                                            int num_blocks, void* k_ws, void* v_ws, int B, int Hkv, int Sq, int D,
                                            int pos0_max, const int32_t* pos0_dev, int window, const float* table,
                                            hipStream_t st);
// Append only: Sq new rows per (batch, KV head) at per-sequence positions pos[b] (device int32
// [B]) into the contiguous cache [B*Hkv, S_max, D] (block_table == nullptr) or the pool
// [num_blocks, Hkv, 1 << bs_log2, D]; keys rotated when table != nullptr.  Sequences with a
// position outside [0, s_cap - Sq] are not written.
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_dst, void* v_dst, const int32_t* pos,
                            int B, int Hkv, int Sq, int D, int S_max, int s_cap, const int32_t* block_table,
                            int max_blocks, int bs_log2, int num_blocks, const float* table, hipStream_t st);
// The attention of a chunk against the cache: a.k holds the fp16 keys (a.table != nullptr) or
// the bf16 cache keys (no RoPE).
hipError_t launch_prefill_cache(const PrefillArgs& a, hipStream_t st);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cache_len;
  const int32_t* q_pos;
  void* o;
  float* lse;
  bool out_bf16;
  int B, Hq, Hkv, S_max, D;
  const float* table;  // nullptr: no RoPE
  int table_max_pos;
  int n_split;
  int chunk;           // keys per split (multiple of the kernel's key block)
  float* ws_o;         // [B, Hq, n_split, D]
  float* ws_ml;        // [B, Hq, n_split, 2]
  // Paged cache (block_table != nullptr): k and v are pools [num_blocks, Hkv, 1 << bs_log2, D];
  // token t of sequence b is in block block_table[b * max_blocks + (t >> bs_log2)];
  // S_max = max_blocks << bs_log2.
  const int32_t* block_table;
  int max_blocks, bs_log2, num_blocks;
  // Sliding window: cache row j is visible only if j >= q_pos[b] - window (no window: 1 << 30).
  int window;
};

constexpr int kNoWindow = 1 << 30;

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
// More than 16 query heads per KV head: K/V tiles shared through LDS.  Usable when
// decode_wide_fits(a): the cache of one sequence (contiguous) or the pool (paged) is under 2 GiB.
bool decode_wide_fits(const DecodeArgs& a);
hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t st);
// The merge pass over a.n_split partials in a.ws_o / a.ws_ml.
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t st);

}  // namespace attn
