// C ABI of libattn.so (declared in include/attn.h): argument validation and kernel dispatch.
//
// Every check that can run on the host runs before the first HIP call, so a rejected call
// enqueues nothing and touches no device state.
#include "../../include/attn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "common.h"

namespace {

constexpr int kVersion = 20200;  // 2.2.0
#ifdef ATTN_CHECKED
constexpr int kCheckedWords = 6;  // source files with index checks (attn_checked_sites)
#endif

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

inline bool valid_dtype(attn_dtype d) { return d == ATTN_F32 || d == ATTN_BF16; }

// window < 0: none; window >= 0: W keys before each query (causal attention only).
inline bool valid_window(int window, bool causal) { return window < 0 || causal; }
inline int kernel_window(int window) { return window < 0 || window >= attn::kNoWindow ? attn::kNoWindow : window; }

attn_status check_rope(const float* table, int table_max_pos, int pos0, int S) {
  if (!table) return ATTN_OK;
  if (!aligned16(table) || table_max_pos < 1 || pos0 < 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)pos0 + S > (int64_t)table_max_pos) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Decode split geometry: keys per split are a multiple of the 32-key wave block.  A unit is a
// (sequence, KV head, group of up to 16 query heads) triple: one workgroup per unit and split.
void decode_geometry(int B, int Hq, int Hkv, int S_max, int n_split_req, int* n_split, int* chunk) {
  const int G = Hq / Hkv;
  int ns = n_split_req;
  if (ns <= 0) {
    int64_t want;
    if (G <= 16) {
      // With >= 256 units, one 8-wave workgroup per unit streams the whole cache and writes o
      // directly (no merge pass).  Below that, split the cache over 4-wave workgroups, aiming
      // for >= 512 of them (2 per CU) with >= 256 keys per split.  Measured on batch 32 x 8 KV
      // heads x 8192 keys: one split, 158 us; 2 splits + merge, 165 us; 4, 168 us.
      const int64_t units = (int64_t)B * Hkv;
      want = units >= 256 ? 1 : (512 + units - 1) / units;
    } else {
      // Wide groups: one workgroup per (sequence, KV head, up to 64 query heads) holds 128 KiB
      // of LDS stages, so one runs per CU; aim for >= 256 of them.
      const int hg = G <= 32 ? 2 : 4;
      const int64_t units = (int64_t)B * Hkv * (((G + 15) / 16 + hg - 1) / hg);
      want = units >= 256 ? 1 : (256 + units - 1) / units;
    }
    int64_t cap = S_max / 256;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    ns = (int)want;
  }
  const int align = G <= 16 ? 32 : 64;
  int c = (S_max + ns - 1) / ns;
  c = ((c + align - 1) / align) * align;
  // drop splits that would start past S_max
  int ns_eff = (S_max + c - 1) / c;
  if (ns_eff < 1) ns_eff = 1;
  *n_split = ns_eff;
  *chunk = c;
}

// Host checks of attn_decode's arguments other than the workspace.
attn_status check_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* cache_len,
                         const int32_t* q_pos, const void* o, const float* lse, attn_dtype in_dt,
                         attn_dtype out_dt, int B, int Hq, int Hkv, int S_max, int D, int window,
                         const float* rope_table, int table_max_pos, int n_split) {
  if (!q || !k_cache || !v_cache || !cache_len || !o) return ATTN_ERR_INVALID_ARG;
  if ((rope_table || window >= 0) && !q_pos) return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || S_max < 1 || D < 1 || n_split < 0) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      (lse && !aligned16(lse)) || (reinterpret_cast<uintptr_t>(cache_len) & 3u) ||
      (q_pos && (reinterpret_cast<uintptr_t>(q_pos) & 3u)))
    return ATTN_ERR_INVALID_ARG;
  if (rope_table && (!aligned16(rope_table) || table_max_pos < 1)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Host checks that follow the workspace check (the support matrix).
attn_status check_decode_support(attn_dtype in_dt, int B, int Hkv, int S_max, int D) {
  if (in_dt != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * S_max * D > (int64_t)1 << 40) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

hipError_t launch_decode_contiguous(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* cache_len, const int32_t* q_pos, void* o, float* lse,
                                    attn_dtype out_dt, int B, int Hq, int Hkv, int S_max, int D, int window,
                                    const float* rope_table, int table_max_pos, int n_split, void* workspace,
                                    hipStream_t st) {
  int ns, chunk;
  decode_geometry(B, Hq, Hkv, S_max, n_split, &ns, &chunk);
  attn::DecodeArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache;
  a.cache_len = cache_len; a.q_pos = q_pos;
  a.o = o; a.lse = lse;
  a.out_bf16 = out_dt == ATTN_BF16;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S_max = S_max; a.D = D;
  a.table = rope_table; a.table_max_pos = table_max_pos;
  a.n_split = ns; a.chunk = chunk;
  const size_t parts = (size_t)B * Hq * ns;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = static_cast<float*>(workspace) + parts * D;
  a.block_table = nullptr;
  a.max_blocks = 0; a.bs_log2 = 0; a.num_blocks = 0;
  a.window = kernel_window(window);
  return attn::launch_decode(a, st);
}

// ---- the static scratch buffer of attn_decode_noalloc --------------------------------------
// One copy per GPU, allocated when the code object is loaded and held until the process ends.
// In host code `scratch` is only the runtime's handle for the symbol: its device address, which
// differs per GPU, is looked up once per device and used everywhere instead.
static_assert(ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch` (nullptr on a HIP error).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int attn_version(void) { return kVersion; }

int attn_checked_sites(unsigned int* words, int n) {
#ifdef ATTN_CHECKED
  const unsigned int w[kCheckedWords] = {attn::checked_word_rope(),         attn::checked_word_cache(),
                                         attn::checked_word_prefill_bf16(), attn::checked_word_prefill_f32(),
                                         attn::checked_word_decode(),       attn::checked_word_decode_wide()};
  for (int i = 0; words && i < n && i < kCheckedWords; ++i) words[i] = w[i];
  return kCheckedWords;
#else
  (void)words;
  (void)n;
  return -1;
#endif
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: outside the support matrix";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error at launch";
  }
  return "unknown attn_status";
}

size_t attn_rope_table_bytes(int max_pos, int D) {
  if (max_pos < 1 || D < 2 || (D & 1)) return 0;
  return (size_t)max_pos * (size_t)D * sizeof(float);
}

attn_status attn_rope_table_init(float* table, int max_pos, int D, double base, void* stream) {
  return attn_rope_table_init_scaled(table, max_pos, D, base, ATTN_ROPE_PLAIN, 1.0, 1, 32.0, 1.0, stream);
}

attn_status attn_rope_table_init_scaled(float* table, int max_pos, int D, double base, attn_rope_scaling scaling,
                                        double factor, int original_max_pos, double beta_fast,
                                        double beta_slow, void* stream) {
  if (!table || !aligned16(table) || max_pos < 1 || D < 2 || (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!(base > 1.0) || !std::isfinite(base)) return ATTN_ERR_INVALID_ARG;
  attn::RopeScalingArgs sc;
  sc.kind = attn::kRopePlain;
  sc.factor = 1.0;
  sc.original_max_pos = 1.0;
  sc.beta_fast = 32.0;
  sc.beta_slow = 1.0;
  if (scaling != ATTN_ROPE_PLAIN) {
    if (scaling != ATTN_ROPE_PI && scaling != ATTN_ROPE_NTK && scaling != ATTN_ROPE_YARN) return ATTN_ERR_INVALID_ARG;
    if (!(factor >= 1.0) || !std::isfinite(factor)) return ATTN_ERR_INVALID_ARG;
    if (scaling == ATTN_ROPE_NTK && D < 4) return ATTN_ERR_INVALID_ARG;
    if (scaling == ATTN_ROPE_YARN &&
        (original_max_pos < 1 || !std::isfinite(beta_fast) || !std::isfinite(beta_slow) || !(beta_fast > beta_slow)))
      return ATTN_ERR_INVALID_ARG;
    sc.kind = scaling == ATTN_ROPE_PI ? attn::kRopePI : (scaling == ATTN_ROPE_NTK ? attn::kRopeNTK : attn::kRopeYaRN);
    sc.factor = factor;
    sc.original_max_pos = (double)original_max_pos;
    sc.beta_fast = beta_fast;
    sc.beta_slow = beta_slow;
  }
  return from_hip(attn::launch_rope_table(table, max_pos, D, base, sc, (hipStream_t)stream));
}

attn_status attn_rope_apply(const void* x, void* out, attn_dtype dt, int B, int H, int S, int D,
                            int pos0, const float* rope_table, int table_max_pos, void* stream) {
  if (!x || !out || !rope_table) return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || S < 1 || D < 2 || (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out)) return ATTN_ERR_INVALID_ARG;
  if (check_rope(rope_table, table_max_pos, pos0, S) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)B * H * S;
  return from_hip(attn::launch_rope_apply(x, out, dt == ATTN_BF16, rows, S, D, pos0, rope_table,
                                          (hipStream_t)stream));
}

size_t attn_prefill_workspace_bytes(int B, int Hkv, int S, int D) {
  if (B < 1 || Hkv < 1 || S < 1 || D < 1) return 0;
  return attn::prefill_workspace_bytes(B, Hkv, S, D);
}

attn_status attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                         attn_dtype in_dt, attn_dtype out_dt, int B, int Hq, int Hkv, int S, int D,
                         int causal, int pos0, int window, const float* rope_table, int table_max_pos,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!valid_window(window, causal != 0)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return ATTN_ERR_INVALID_ARG;
  if (check_rope(rope_table, table_max_pos, pos0, S) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (workspace && (!aligned16(workspace) ||
                    workspace_bytes < attn::prefill_workspace_bytes(B, Hkv, S, D)))
    return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (in_dt == ATTN_F32 && out_dt != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * S > (int64_t)INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;

  attn::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.out_bf16 = out_dt == ATTN_BF16;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.D = D;
  a.Sk = S; a.k_rows = S; a.v_rows = S; a.coff = 0;
  a.window = kernel_window(window);
  a.causal = causal != 0;
  a.pos0 = pos0;
  a.table = rope_table;
  a.workspace = (rope_table && in_dt == ATTN_BF16) ? workspace : nullptr;
  hipStream_t st = (hipStream_t)stream;
  return from_hip(in_dt == ATTN_F32 ? attn::launch_prefill_f32(a, st) : attn::launch_prefill_bf16(a, st));
}

attn_status attn_rotate_keys_f16(const void* k, void* k_rot, int B, int Hkv, int S, int D, int pos0,
                                 const float* rope_table, int table_max_pos, void* stream) {
  if (!k || !k_rot || !rope_table) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || S < 1 || D < 1 || (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(k_rot)) return ATTN_ERR_INVALID_ARG;
  if (check_rope(rope_table, table_max_pos, pos0, S) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  return from_hip(attn::launch_rotate_keys_f16(k, k_rot, B, Hkv, S, D, pos0, rope_table, (hipStream_t)stream));
}

attn_status attn_prefill_prerotated(const void* q, const void* k_rot, const void* v, void* o, float* lse,
                                    attn_dtype out_dt, int B, int Hq, int Hkv, int S, int D, int causal,
                                    int pos0, int window, const float* rope_table, int table_max_pos,
                                    void* stream) {
  if (!q || !k_rot || !v || !o || !rope_table) return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(out_dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1 || (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!valid_window(window, causal != 0)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_rot) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return ATTN_ERR_INVALID_ARG;
  if (check_rope(rope_table, table_max_pos, pos0, S) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * S > (int64_t)INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  attn::PrefillArgs a;
  a.q = q; a.k = k_rot; a.v = v; a.o = o; a.lse = lse;
  a.out_bf16 = out_dt == ATTN_BF16;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.D = D;
  a.Sk = S; a.k_rows = S; a.v_rows = S; a.coff = 0;
  a.window = kernel_window(window);
  a.causal = causal != 0;
  a.pos0 = pos0;
  a.table = rope_table;
  a.workspace = nullptr;
  return from_hip(attn::launch_prefill_prerotated(a, k_rot, (hipStream_t)stream));
}

attn_status attn_prefill_chunk(const void* q, const void* k_new, const void* v_new, void* k_cache,
                               void* v_cache, void* o, float* lse, attn_dtype out_dt, int B, int Hq,
                               int Hkv, int Sq, int S_max, int D, int pos0, int window,
                               const float* rope_table, int table_max_pos, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !o) return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(out_dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || S_max < 1 || D < 1 || pos0 < 0) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)pos0 + Sq > (int64_t)S_max) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(o) || (lse && !aligned16(lse)))
    return ATTN_ERR_INVALID_ARG;
  if (check_rope(rope_table, table_max_pos, pos0, Sq) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  const int Sk = pos0 + Sq;
  if (rope_table && (!workspace || !aligned16(workspace) ||
                     workspace_bytes < attn::prefill_workspace_bytes(B, Hkv, Sk, D)))
    return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * Sq > (int64_t)INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;

  hipStream_t st = (hipStream_t)stream;
  void* k16 = rope_table ? workspace : nullptr;
  const int kw = kernel_window(window);
  // key rows the attention can still read: from the 64-key tile holding the first row's window start
  const int conv_first = kw >= pos0 ? 0 : ((pos0 - kw) / 64) * 64;
  const hipError_t e = attn::launch_cache_append(k_new, v_new, k_cache, v_cache, k16, B, Hkv, Sq, S_max,
                                                 D, pos0, conv_first, rope_table, st);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  attn::PrefillArgs a;
  a.q = q; a.k = rope_table ? k16 : k_cache; a.v = v_cache; a.o = o; a.lse = lse;
  a.out_bf16 = out_dt == ATTN_BF16;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = Sq; a.D = D;
  a.causal = true;
  a.pos0 = pos0;
  a.table = rope_table;
  a.workspace = nullptr;
  a.Sk = Sk; a.k_rows = rope_table ? Sk : S_max; a.v_rows = S_max; a.coff = pos0;
  a.window = kw;
  return from_hip(attn::launch_prefill_cache(a, st));
}

attn_status attn_prefill_chunk_varpos(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, const int32_t* pos0, int pos0_max, void* o, float* lse,
                                      attn_dtype out_dt, int B, int Hq, int Hkv, int Sq, int S_max, int D,
                                      int window, const float* rope_table, int table_max_pos,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !o || !pos0) return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(out_dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || S_max < 1 || D < 1 || pos0_max < 0) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)pos0_max + Sq > (int64_t)S_max) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(o) || (lse && !aligned16(lse)) || (reinterpret_cast<uintptr_t>(pos0) & 3u))
    return ATTN_ERR_INVALID_ARG;
  if (check_rope(rope_table, table_max_pos, pos0_max, Sq) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  const int Sk_max = pos0_max + Sq;
  if (rope_table && (!workspace || !aligned16(workspace) ||
                     workspace_bytes < attn::prefill_workspace_bytes(B, Hkv, Sk_max, D)))
    return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * Sq > (int64_t)INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;

  hipStream_t st = (hipStream_t)stream;
  void* k16 = rope_table ? workspace : nullptr;
  const int kw = kernel_window(window);
  // each sequence's start is read on the device; pos0_max bounds them and sizes the fp16 rows
  const hipError_t e = attn::launch_cache_append_varpos(k_new, v_new, k_cache, v_cache, k16, B, Hkv, Sq, S_max,
                                                        D, pos0_max, pos0, kw, rope_table, st);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  attn::PrefillArgs a;
  a.q = q; a.k = rope_table ? k16 : k_cache; a.v = v_cache; a.o = o; a.lse = lse;
  a.out_bf16 = out_dt == ATTN_BF16;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = Sq; a.D = D;
  a.causal = true;
  a.pos0 = pos0_max;
  a.table = rope_table;
  a.workspace = nullptr;
  a.Sk = Sk_max; a.k_rows = rope_table ? Sk_max : S_max; a.v_rows = S_max; a.coff = pos0_max;
  a.window = kw;
  a.pos0_dev = pos0;
  return from_hip(attn::launch_prefill_cache(a, st));
}

size_t attn_prefill_chunk_paged_workspace_bytes(int B, int Hkv, int pos0, int Sq, int D) {
  if (B < 1 || Hkv < 1 || pos0 < 0 || Sq < 1 || D < 1) return 0;
  // the keys (with their exponent bytes) of the visible rows, then their values
  return attn::prefill_workspace_bytes(B, Hkv, pos0 + Sq, D) + attn::prefill_kexp_offset(B, Hkv, pos0 + Sq, D);
}

attn_status attn_prefill_chunk_paged(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                     void* v_pages, int num_blocks, int block_size, const int32_t* block_table,
                                     int max_blocks, void* o, float* lse, attn_dtype out_dt, int B, int Hq,
                                     int Hkv, int Sq, int D, int pos0, int window, const float* rope_table,
                                     int table_max_pos, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_new || !v_new || !k_pages || !v_pages || !block_table || !o || !workspace)
    return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(out_dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || D < 1 || pos0 < 0 || num_blocks < 1 || max_blocks < 1)
    return ATTN_ERR_INVALID_ARG;
  if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)max_blocks * block_size > (int64_t)INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)pos0 + Sq > (int64_t)max_blocks * block_size) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages) || !aligned16(v_pages) ||
      !aligned16(o) || !aligned16(workspace) || (lse && !aligned16(lse)) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return ATTN_ERR_INVALID_ARG;
  if (check_rope(rope_table, table_max_pos, pos0, Sq) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn_prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D)) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * Sq > (int64_t)INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)num_blocks * Hkv * block_size * D > (int64_t)1 << 40) return ATTN_ERR_UNSUPPORTED;

  hipStream_t st = (hipStream_t)stream;
  const int Sk = pos0 + Sq;
  void* k_ws = workspace;
  void* v_ws = static_cast<char*>(workspace) + attn::prefill_workspace_bytes(B, Hkv, Sk, D);
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  const int kw = kernel_window(window);
  // rows the attention can still read: from the 64-key tile holding the first row's window start
  const int conv_first = kw >= pos0 ? 0 : ((pos0 - kw) / 64) * 64;
  const int first_seen = kw >= pos0 ? 0 : pos0 - kw;  // the first query's window start
  const hipError_t e = attn::launch_cache_append_paged(k_new, v_new, k_pages, v_pages, block_table, max_blocks,
                                                       bs_log2, num_blocks, k_ws, v_ws, B, Hkv, Sq, D, pos0,
                                                       conv_first, first_seen, rope_table, st);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  attn::PrefillArgs a;
  a.q = q; a.k = k_ws; a.v = v_ws; a.o = o; a.lse = lse;
  a.out_bf16 = out_dt == ATTN_BF16;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = Sq; a.D = D;
  a.causal = true;
  a.pos0 = pos0;
  a.table = rope_table;
  a.workspace = nullptr;
  a.Sk = Sk; a.k_rows = Sk; a.v_rows = Sk; a.coff = pos0;
  a.window = kw;
  return from_hip(attn::launch_prefill_cache(a, st));
}

attn_status attn_prefill_chunk_paged_varpos(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                            void* v_pages, int num_blocks, int block_size,
                                            const int32_t* block_table, int max_blocks, const int32_t* pos0,
                                            int pos0_max, void* o, float* lse, attn_dtype out_dt, int B, int Hq,
                                            int Hkv, int Sq, int D, int window, const float* rope_table,
                                            int table_max_pos, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  if (!q || !k_new || !v_new || !k_pages || !v_pages || !block_table || !pos0 || !o || !workspace)
    return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(out_dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || D < 1 || pos0_max < 0 || num_blocks < 1 || max_blocks < 1)
    return ATTN_ERR_INVALID_ARG;
  if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)max_blocks * block_size > (int64_t)INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)pos0_max + Sq > (int64_t)max_blocks * block_size) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages) || !aligned16(v_pages) ||
      !aligned16(o) || !aligned16(workspace) || (lse && !aligned16(lse)) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(pos0) & 3u))
    return ATTN_ERR_INVALID_ARG;
  if (check_rope(rope_table, table_max_pos, pos0_max, Sq) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn_prefill_chunk_paged_workspace_bytes(B, Hkv, pos0_max, Sq, D))
    return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * Sq > (int64_t)INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)num_blocks * Hkv * block_size * D > (int64_t)1 << 40) return ATTN_ERR_UNSUPPORTED;

  hipStream_t st = (hipStream_t)stream;
  const int Sk_max = pos0_max + Sq;
  void* k_ws = workspace;
  void* v_ws = static_cast<char*>(workspace) + attn::prefill_workspace_bytes(B, Hkv, Sk_max, D);
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  const int kw = kernel_window(window);
  // each sequence's start is read on the device; its rows are gathered from its own window start
  const hipError_t e = attn::launch_cache_append_paged_varpos(k_new, v_new, k_pages, v_pages, block_table,
                                                              max_blocks, bs_log2, num_blocks, k_ws, v_ws, B, Hkv,
                                                              Sq, D, pos0_max, pos0, kw, rope_table, st);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  attn::PrefillArgs a;
  a.q = q; a.k = k_ws; a.v = v_ws; a.o = o; a.lse = lse;
  a.out_bf16 = out_dt == ATTN_BF16;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = Sq; a.D = D;
  a.causal = true;
  a.pos0 = pos0_max;
  a.table = rope_table;
  a.workspace = nullptr;
  a.Sk = Sk_max; a.k_rows = Sk_max; a.v_rows = Sk_max; a.coff = pos0_max;
  a.window = kw;
  a.pos0_dev = pos0;
  return from_hip(attn::launch_prefill_cache(a, st));
}

attn_status attn_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* pos, int B, int Hkv, int Sq, int S_max, int D,
                              const float* rope_table, int table_max_pos, void* stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !pos) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || Sq < 1 || S_max < 1 || D < 1 || Sq > S_max) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(pos) & 3u))
    return ATTN_ERR_INVALID_ARG;
  if (rope_table && (!aligned16(rope_table) || table_max_pos < Sq)) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * S_max * D > (int64_t)1 << 40) return ATTN_ERR_UNSUPPORTED;
  const int s_cap = rope_table ? std::min(S_max, table_max_pos) : S_max;
  return from_hip(attn::launch_kv_append(k_new, v_new, k_cache, v_cache, pos, B, Hkv, Sq, D, S_max, s_cap, nullptr,
                                         0, 0, 0, rope_table, (hipStream_t)stream));
}

attn_status attn_cache_append_paged(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                                    int num_blocks, int block_size, const int32_t* block_table, int max_blocks,
                                    const int32_t* pos, int B, int Hkv, int Sq, int D, const float* rope_table,
                                    int table_max_pos, void* stream) {
  if (!k_new || !v_new || !k_pages || !v_pages || !block_table || !pos) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || Sq < 1 || D < 1 || num_blocks < 1 || max_blocks < 1) return ATTN_ERR_INVALID_ARG;
  if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)max_blocks * block_size > (int64_t)INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)Sq > (int64_t)max_blocks * block_size) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages) || !aligned16(v_pages) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(pos) & 3u))
    return ATTN_ERR_INVALID_ARG;
  if (rope_table && (!aligned16(rope_table) || table_max_pos < Sq)) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)num_blocks * Hkv * block_size * D > (int64_t)1 << 40) return ATTN_ERR_UNSUPPORTED;
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  const int cap = max_blocks * block_size;
  const int s_cap = rope_table ? std::min(cap, table_max_pos) : cap;
  return from_hip(attn::launch_kv_append(k_new, v_new, k_pages, v_pages, pos, B, Hkv, Sq, D, 0, s_cap, block_table,
                                         max_blocks, bs_log2, num_blocks, rope_table, (hipStream_t)stream));
}

int attn_decode_num_splits(int B, int Hq, int Hkv, int S_max, int D, int n_split) {
  (void)D;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S_max < 1 || n_split < 0) return 0;
  int ns, chunk;
  decode_geometry(B, Hq, Hkv, S_max, n_split, &ns, &chunk);
  return ns;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int S_max, int D, int n_split) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S_max < 1 || D < 1 || n_split < 0) return 0;
  int ns, chunk;
  decode_geometry(B, Hq, Hkv, S_max, n_split, &ns, &chunk);
  const size_t parts = (size_t)B * Hq * ns;
  return parts * (size_t)D * sizeof(float) + parts * 2 * sizeof(float);
}

attn_status attn_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cache_len, const int32_t* q_pos, void* o, float* lse,
                        attn_dtype in_dt, attn_dtype out_dt, int B, int Hq, int Hkv, int S_max,
                        int D, int window, const float* rope_table, int table_max_pos, int n_split,
                        void* workspace, size_t workspace_bytes, void* stream) {
  attn_status s = check_decode(q, k_cache, v_cache, cache_len, q_pos, o, lse, in_dt, out_dt, B, Hq, Hkv, S_max,
                               D, window, rope_table, table_max_pos, n_split);
  if (s != ATTN_OK) return s;
  if (!workspace || !aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn_decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split))
    return ATTN_ERR_INVALID_ARG;
  s = check_decode_support(in_dt, B, Hkv, S_max, D);
  if (s != ATTN_OK) return s;
  return from_hip(launch_decode_contiguous(q, k_cache, v_cache, cache_len, q_pos, o, lse, out_dt, B, Hq, Hkv,
                                           S_max, D, window, rope_table, table_max_pos, n_split, workspace,
                                           (hipStream_t)stream));
}

attn_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* cache_len, const int32_t* q_pos, void* o, float* lse,
                                attn_dtype in_dt, attn_dtype out_dt, int B, int Hq, int Hkv, int S_max, int D,
                                int window, const float* rope_table, int table_max_pos, int n_split,
                                void* stream) {
  attn_status s = check_decode(q, k_cache, v_cache, cache_len, q_pos, o, lse, in_dt, out_dt, B, Hq, Hkv, S_max,
                               D, window, rope_table, table_max_pos, n_split);
  if (s != ATTN_OK) return s;
  // the partials of every split must fit the static buffer
  if (attn_decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    return ATTN_ERR_UNSUPPORTED;
  s = check_decode_support(in_dt, B, Hkv, S_max, D);
  if (s != ATTN_OK) return s;
  void* ptr = scratch_on_current_device();
  if (!ptr) return ATTN_ERR_HIP;
  return from_hip(launch_decode_contiguous(q, k_cache, v_cache, cache_len, q_pos, o, lse, out_dt, B, Hq, Hkv,
                                           S_max, D, window, rope_table, table_max_pos, n_split, ptr,
                                           (hipStream_t)stream));
}

attn_status attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, int num_blocks,
                              int block_size, const int32_t* block_table, int max_blocks,
                              const int32_t* cache_len, const int32_t* q_pos, void* o, float* lse,
                              attn_dtype in_dt, attn_dtype out_dt, int B, int Hq, int Hkv, int D, int window,
                              const float* rope_table, int table_max_pos, int n_split, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !cache_len || !o || !workspace) return ATTN_ERR_INVALID_ARG;
  if ((rope_table || window >= 0) && !q_pos) return ATTN_ERR_INVALID_ARG;
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || num_blocks < 1 || max_blocks < 1 || n_split < 0)
    return ATTN_ERR_INVALID_ARG;
  if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)max_blocks * block_size > (int64_t)INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (rope_table && (D & 1)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) || !aligned16(workspace) ||
      (lse && !aligned16(lse)) || (reinterpret_cast<uintptr_t>(cache_len) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (q_pos && (reinterpret_cast<uintptr_t>(q_pos) & 3u)))
    return ATTN_ERR_INVALID_ARG;
  if (rope_table && (!aligned16(rope_table) || table_max_pos < 1)) return ATTN_ERR_INVALID_ARG;
  const int S_max = max_blocks * block_size;
  if (workspace_bytes < attn_decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split)) return ATTN_ERR_INVALID_ARG;
  if (in_dt != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)num_blocks * Hkv * block_size * D > (int64_t)1 << 40) return ATTN_ERR_UNSUPPORTED;

  int ns, chunk;
  decode_geometry(B, Hq, Hkv, S_max, n_split, &ns, &chunk);
  attn::DecodeArgs a;
  a.q = q; a.k = k_pages; a.v = v_pages;
  a.cache_len = cache_len; a.q_pos = q_pos;
  a.o = o; a.lse = lse;
  a.out_bf16 = out_dt == ATTN_BF16;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S_max = S_max; a.D = D;
  a.table = rope_table; a.table_max_pos = table_max_pos;
  a.n_split = ns; a.chunk = chunk;
  const size_t parts = (size_t)B * Hq * ns;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = static_cast<float*>(workspace) + parts * D;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  a.bs_log2 = lg;
  a.num_blocks = num_blocks;
  a.window = kernel_window(window);
  return from_hip(attn::launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"
