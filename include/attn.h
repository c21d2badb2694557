/*
 * attn.h -- C ABI of libattn.so: rotary position embeddings and exact causal multi-head /
 * grouped-query scaled dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * What is computed (all citations name a page and its section):
 *
 *   RoPE      "Transformer Architecture & Self-Attention Mechanics" (devthesis.com),
 *             section 3, "Rotary Position Embeddings (RoPE)": the head vector is cut into
 *             adjacent pairs (x[2i], x[2i+1]); at position m pair i is turned
 *             counter-clockwise by m * theta_i, theta_i = base^(-2i/D).
 *   Attention same page, section 1, the "Attention(Q,K,V)" equation with the row-wise
 *             softmax; scale 1/sqrt(D).  Causal masking as in the PyTorch listing of
 *             "Multi-Head Attention & Rotary Position Embeddings (RoPE)"
 *             (learnllm.online): key j is visible to query i only if j <= i.
 *   Tiling    "Building Self-Attention and Transformer Engines" (codingpancake.com),
 *             section 4.1 / 4.2: the S x S score matrix is never written to memory; the
 *             softmax is accumulated tile by tile with a running max and sum.
 *   GQA       same page, section 6.1 and the comparison table of section 7: a group of
 *             G = Hq / Hkv query heads shares one K/V head; query head h reads KV head
 *             h / G (integer division).
 *   Decode    "Transformer internals: attention without the mysticism"
 *             (ninaddeshpande.com), "The KV cache and the memory wall": one new query per
 *             sequence against the cached keys and values.
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, row-major ("C order") [B, H, S, D] with D innermost, on the
 *     device.  Every tensor pointer must be 16-byte aligned.
 *   - The caller owns all memory.  The library allocates nothing, keeps no state between
 *     calls (attn_decode_noalloc's static buffer aside), never synchronises, and enqueues its kernels on `stream` (a hipStream_t;
 *     NULL means the default stream).  Calls are asynchronous: a returned ATTN_OK means
 *     the work was enqueued.
 *   - Only kernel launches reach the stream (no memset, copy or event), so a call made
 *     while the stream is being captured into a HIP graph is captured whole and can be
 *     replayed; its buffers must then stay allocated for as long as the graph is used.
 *   - Every argument that can be checked on the host is checked before any HIP call; a
 *     rejected call enqueues nothing.  HIP launch errors map to ATTN_ERR_HIP.
 *   - No C++ exception crosses this interface.  Calls are thread-safe (no shared state),
 *     except attn_decode_noalloc, whose calls on one GPU share that GPU's static buffer.
 *   - window (every attention entry point): a negative value means no window.  window = W >= 0
 *     is a sliding window ("Building Self-Attention and Transformer Engines",
 *     codingpancake.com, section 6.4: each token attends only to the W tokens before it): the
 *     query at position p sees only the keys at positions p - W .. p.  It requires the causal
 *     mask.  W = 4096 is the page's example.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, table too short, ... */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request outside the support matrix (head dim, dtype) */
  ATTN_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} attn_status;

/* The enumerations taken as arguments span every int (their _RANGE_ members), so that any int
 * a caller passes is a value of the type; those outside the named ones are rejected with
 * ATTN_ERR_INVALID_ARG. */
typedef enum {
  ATTN_F32 = 0,  /* IEEE binary32 */
  ATTN_BF16 = 1, /* bfloat16; results are rounded to nearest, ties to even */
  ATTN_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  ATTN_DTYPE_RANGE_MAX_ = 2147483647
} attn_dtype;

/* Version of this interface (major * 10000 + minor * 100 + patch).  2.0.0: the buffer of
 * attn_rotate_keys_f16 holds one exponent byte per key row after the rotated keys; 2.1.0:
 * attn_checked_sites; 2.2.0: attn_prefill_chunk_varpos, attn_prefill_chunk_paged_varpos,
 * attn_cache_append and attn_cache_append_paged. */
int attn_version(void);

/* Index checks of a checked build (the library compiled with ATTN_CHECKED; a debugging aid, not
 * the product build).  There every kernel tests the largest index each thread is about to use
 * against the extents its arguments give; a failed test sets a bit in a per-source-file word
 * and the thread skips the accesses it guards instead of faulting.  This call copies up to n of
 * those words into words (when not NULL), in the order rope, cache, prefill_bf16, prefill_f32,
 * decode, decode_wide (bit i of a word: check site i of that file, named in its source), clears
 * them, and returns the number of words (6).  The copies are blocking: call it once the work
 * checked has completed, with no other call on the device in flight.  A normal build returns -1
 * and touches nothing. */
int attn_checked_sites(unsigned int* words, int n);

/* Human-readable name of a status code (static string, never NULL).  Any int is accepted; a value
 * that is no attn_status gives "unknown attn_status". */
const char* attn_status_string(int status);

/* ---------------------------------------------------------------------------------------
 * RoPE coefficient table.
 *
 * Layout: float32 [max_pos][D/2][2]; entry (m, i) holds cos(m * theta_i) then
 * sin(m * theta_i), theta_i = base^(-2i/D) (devthesis section 3).  The angle m * theta_i
 * is formed in double precision and its cosine and sine are rounded once to float32.
 * attn_rope_table_bytes returns the size in bytes (0 if max_pos < 1, D < 2 or D is odd).
 * attn_rope_table_init fills a caller-allocated device buffer of that size.
 * Errors: ATTN_ERR_INVALID_ARG for table == NULL, max_pos < 1, odd D or D < 2,
 * base <= 1, or a table not 16-byte aligned.
 * --------------------------------------------------------------------------------------- */
size_t attn_rope_table_bytes(int max_pos, int D);
attn_status attn_rope_table_init(float* table, int max_pos, int D, double base, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_rope_table_init_scaled: the same table with a frequency scaling for contexts longer
 * than the trained one.  The pages name Position Interpolation, NTK-aware scaling and YaRN
 * ("Transformer internals: attention without the mysticism", ninaddeshpande.com, "Rotary
 * positional embeddings (RoPE)"; devthesis.com Problem 3, "Superiority for Context Window
 * Extension") without formulas; these follow the methods' publications, with s = factor:
 *   ATTN_ROPE_PLAIN  the plain table (factor and the rest ignored);
 *   ATTN_ROPE_PI     angle (m / s) * theta_i;
 *   ATTN_ROPE_NTK    theta_i from the base base * s^(D / (D - 2)) (D >= 4);
 *   ATTN_ROPE_YARN   with r_i = original_max_pos * theta_i / (2 pi) and
 *                    g_i = clamp((r_i - beta_slow) / (beta_fast - beta_slow), 0, 1):
 *                    theta_i' = (1 - g_i) theta_i / s + g_i theta_i, and entries scaled by
 *                    0.1 ln(s) + 1 (so scores by its square); usual betas 32 and 1.
 * Every kernel reads its rotation from the table, so a scaled table works everywhere a table
 * is taken; keys stored in a KV cache must have been rotated with the same table.
 * Errors: as attn_rope_table_init, plus ATTN_ERR_INVALID_ARG for an unknown scaling,
 * factor < 1 or not finite, NTK with D < 4, YaRN with original_max_pos < 1 or
 * beta_fast <= beta_slow.
 * --------------------------------------------------------------------------------------- */
typedef enum {
  ATTN_ROPE_PLAIN = 0,
  ATTN_ROPE_PI = 1,
  ATTN_ROPE_NTK = 2,
  ATTN_ROPE_YARN = 3,
  ATTN_ROPE_RANGE_MIN_ = -2147483647 - 1,
  ATTN_ROPE_RANGE_MAX_ = 2147483647
} attn_rope_scaling;
attn_status attn_rope_table_init_scaled(float* table, int max_pos, int D, double base,
                                        attn_rope_scaling scaling, double factor, int original_max_pos,
                                        double beta_fast, double beta_slow, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_rope_apply: out[b,h,s,:] = RoPE(x[b,h,s,:]) at position pos0 + s
 * (devthesis section 3; the dim-8 example of "Transformer Architecture: FlashAttention &
 * RoPE", academy.kwas.tech).
 *
 * x, out: [B, H, S, D] of dtype dt; out == x rotates in place, otherwise the buffers must
 * not overlap.  The rotation is computed in float32 with the table's coefficients, then
 * stored as dt.  Any even D >= 2 is accepted.
 * Errors: ATTN_ERR_INVALID_ARG for null pointers, B/H/S < 1, odd D, pos0 < 0,
 * pos0 + S > table_max_pos, or misaligned pointers.
 * --------------------------------------------------------------------------------------- */
attn_status attn_rope_apply(const void* x, void* out, attn_dtype dt, int B, int H, int S, int D,
                            int pos0, const float* rope_table, int table_max_pos, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_prefill: exact attention of S queries against the same S keys, tiled with an
 * online softmax (codingpancake section 4).
 *
 * q: [B, Hq, S, D]; k, v: [B, Hkv, S, D], all of dtype in_dt.
 * o: [B, Hq, S, D] of dtype out_dt (written in full).
 * lse: optional float32 [B, Hq, S]; if not NULL receives the natural-log normaliser
 *      m + ln(sum_j exp(s_ij - m)) of the scaled scores of each row.
 * rope_table: NULL disables RoPE; otherwise Q and K rows are rotated at positions
 *      pos0 + s before the product (V is never rotated); requires pos0 >= 0 and
 *      pos0 + S <= table_max_pos.
 * causal != 0 masks key j > query i (square mask anchored at the top-left); causal == 0
 *      lets every query see every key.
 * window: see the conventions above; W >= 0 also masks key j < i - W (needs causal != 0).
 * Scale: 1/sqrt(D), fixed.
 * workspace: optional device scratch of at least attn_prefill_workspace_bytes(B, Hkv, S, D)
 *      bytes (contents on entry irrelevant, overwritten).  Used only for bf16 input with RoPE:
 *      the keys are then rotated once, in one pass, into the workspace (the layout of
 *      attn_rotate_keys_f16), and the attention kernel streams the rotated keys.  With
 *      workspace == NULL the key rotation is fused into every K tile load instead (same
 *      results; more arithmetic per tile).
 *
 * Support matrix: D in {64, 128}; in_dt = ATTN_F32 (float32 arithmetic throughout, out_dt
 * must be ATTN_F32) or in_dt = ATTN_BF16 (out_dt either).  For bf16 input with RoPE the
 * rotated q and k rows are rounded to IEEE half precision for the Q.K^T matrix-core product
 * (fp32 accumulation).  A row whose largest magnitude reaches 2^15 (a query row after its
 * scale log2(e)/sqrt(D)) is first multiplied by 2^-e, e the smallest non-negative integer
 * that brings it below 2^15, and its products are multiplied by 2^e again in float32: every
 * finite bf16 input has a result as accurate as for small rows, until a score itself leaves
 * the float32 range.  Elements below 2^-14 after that scale are half-precision subnormals
 * (absolute precision 2^-24).  Without RoPE the bf16 inputs are multiplied exactly.  The
 * softmax weights are rounded to bf16 for the P.V product (fp32 accumulation).
 * Errors: ATTN_ERR_INVALID_ARG for null q/k/v/o, B/Hq/Hkv/S < 1, Hq % Hkv != 0, bad RoPE
 * range, a window without the causal mask, a workspace that is misaligned or too small,
 * misalignment; ATTN_ERR_UNSUPPORTED outside the support matrix.
 * --------------------------------------------------------------------------------------- */
size_t attn_prefill_workspace_bytes(int B, int Hkv, int S, int D);
attn_status attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                         attn_dtype in_dt, attn_dtype out_dt, int B, int Hq, int Hkv, int S, int D,
                         int causal, int pos0, int window, const float* rope_table, int table_max_pos,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * The two stages of attn_prefill with a workspace, callable on their own (for example to
 * rotate a sequence's keys once and run several query batches against them).
 *
 * attn_rotate_keys_f16: key row r = RoPE(k[b,h,s,:]) at position pos0 + s, computed in
 *   float32 from bf16 k [B, Hkv, S, D].  k_rot is a device buffer of at least
 *   attn_prefill_workspace_bytes(B, Hkv, S, D) bytes, 16-byte aligned, owned by the caller:
 *   it receives first IEEE half [B, Hkv, S, D] holding r * 2^-e, then one unsigned byte e per
 *   row [B, Hkv, S], where e is the smallest non-negative integer with max |r| * 2^-e < 2^15
 *   (0 for every row below 2^15, and for a row holding an infinity; inf and NaN elements are
 *   stored as they are and propagate to the scores).
 * attn_prefill_prerotated: attn_prefill for bf16 q and v with RoPE, whose keys were already
 *   rotated by attn_rotate_keys_f16 with the same table and pos0 (k_rot is that buffer, read
 *   and never rotated again; q is rotated at pos0 + s).  Other arguments as in attn_prefill.
 * Support matrix: D in {64, 128}.  Errors as in attn_prefill (rope_table is required).
 * --------------------------------------------------------------------------------------- */
attn_status attn_rotate_keys_f16(const void* k, void* k_rot, int B, int Hkv, int S, int D, int pos0,
                                 const float* rope_table, int table_max_pos, void* stream);
attn_status attn_prefill_prerotated(const void* q, const void* k_rot, const void* v, void* o,
                                    float* lse, attn_dtype out_dt, int B, int Hq, int Hkv, int S,
                                    int D, int causal, int pos0, int window, const float* rope_table,
                                    int table_max_pos, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_prefill_chunk: a chunk of Sq new tokens at positions pos0 .. pos0+Sq-1 of every
 * sequence is appended to a KV cache, and its queries attend to the whole cache up to
 * themselves.  The cache keeps earlier tokens' keys and values for reuse (ninaddeshpande.com,
 * "The KV cache and the memory wall"); prefill in chunks is named on learnllm.online,
 * "Prefill vs Decode Latency & Memory Wall Waterfall".
 *
 * q: [B, Hq, Sq, D] (not yet rotated); k_new, v_new: [B, Hkv, Sq, D] (k_new not yet rotated);
 * k_cache, v_cache: [B, Hkv, S_max, D], rows [0, pos0) holding the earlier tokens (keys
 * already rotated, the format attn_decode reads).  All bf16.
 * Step 1 writes cache rows [pos0, pos0 + Sq): key row s = RoPE(k_new row s - pos0) at
 *   position s, computed in float32 and rounded to bf16 (nearest even); value rows copied.
 *   Other cache rows are not modified.
 * Step 2: o[b, h, i] = softmax over keys j <= pos0 + i of the cache rows [0, pos0 + Sq)
 *   (the causal mask aligned at the bottom right), the query rotated at position pos0 + i;
 *   with a window W >= 0 only keys j >= pos0 + i - W.
 *   Query head h reads KV head h / (Hq / Hkv).  Scale 1/sqrt(D).
 * o: [B, Hq, Sq, D] of dtype out_dt; lse: optional float32 [B, Hq, Sq] (natural log).
 * rope_table: NULL disables RoPE (keys copied into the cache as given, Q.K^T on the exact
 *   bf16 values); otherwise requires pos0 + Sq <= table_max_pos.
 * workspace: required with RoPE: at least attn_prefill_workspace_bytes(B, Hkv, pos0 + Sq, D)
 *   bytes, 16-byte aligned, contents irrelevant.  It receives every key row [0, pos0 + Sq) in
 *   the Q.K^T operand format of attn_rotate_keys_f16 (IEEE half with a per-row exponent, so
 *   cached keys of any finite magnitude are handled as in attn_prefill).
 * k_new, v_new and q must not overlap the cache.  pos0 = 0 is an ordinary causal prefill whose
 * keys are kept.
 * Support matrix: D in {64, 128}; out_dt either.
 * Errors: ATTN_ERR_INVALID_ARG for null pointers, sizes < 1, pos0 < 0, pos0 + Sq > S_max,
 * Hq % Hkv != 0, bad RoPE range, missing/small/misaligned workspace with RoPE,
 * misalignment; ATTN_ERR_UNSUPPORTED outside the support matrix.
 * --------------------------------------------------------------------------------------- */
attn_status attn_prefill_chunk(const void* q, const void* k_new, const void* v_new, void* k_cache,
                               void* v_cache, void* o, float* lse, attn_dtype out_dt, int B, int Hq,
                               int Hkv, int Sq, int S_max, int D, int pos0, int window,
                               const float* rope_table, int table_max_pos, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_prefill_chunk_varpos: attn_prefill_chunk for a batch whose sequences have reached
 * different lengths (same page sections): sequence b's chunk of Sq tokens sits at positions
 * p_b .. p_b+Sq-1, p_b = pos0[b], and is appended to its cache rows [p_b, p_b + Sq); its
 * queries attend to cache rows j <= p_b + i (and, with a window W >= 0, j >= p_b + i - W).
 *
 * pos0: device int32 [B], 4-byte aligned, read on the device only.  Each value must lie in
 *   [0, pos0_max].  A sequence whose value lies outside gets NaN output rows (and NaN LSE),
 *   and its cache rows are left unchanged; the other sequences are not affected.
 * pos0_max: host int >= 0, the largest start the call allows: pos0_max + Sq <= S_max, and
 *   with RoPE pos0_max + Sq <= table_max_pos.
 * workspace: required with RoPE: at least attn_prefill_workspace_bytes(B, Hkv, pos0_max + Sq, D)
 *   bytes, 16-byte aligned, contents irrelevant.
 * With every pos0[b] equal to p the result is attn_prefill_chunk's with pos0 = p, bit for bit.
 * Other arguments, layouts, the support matrix and the errors as in attn_prefill_chunk (with
 * pos0_max in place of pos0); also ATTN_ERR_INVALID_ARG for a null or misaligned pos0.
 * --------------------------------------------------------------------------------------- */
attn_status attn_prefill_chunk_varpos(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, const int32_t* pos0, int pos0_max, void* o, float* lse,
                                      attn_dtype out_dt, int B, int Hq, int Hkv, int Sq, int S_max, int D,
                                      int window, const float* rope_table, int table_max_pos,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_prefill_chunk_paged: attn_prefill_chunk against a paged KV cache, the block pool of
 * codingpancake.com "Building Self-Attention and Transformer Engines", section 6.2 (the cache
 * attn_decode_paged reads).
 *
 * k_pages, v_pages: bf16 pools [num_blocks, Hkv, block_size, D]; block_table: device int32
 * [B, max_blocks]; token t of sequence b is stored in block block_table[b * max_blocks +
 * t / block_size], slot t % block_size.  block_size is a power of two in [16, 4096];
 * pos0 + Sq <= max_blocks * block_size.
 * Step 1 writes the slots of tokens pos0 .. pos0+Sq-1 (keys rotated at their positions and
 *   rounded to bf16, values copied) and no other slot.  The blocks receiving them must not be
 *   shared between sequences; blocks holding only earlier tokens may be.
 * Step 2 is attn_prefill_chunk's: o[b, h, i] = softmax over tokens j <= pos0 + i (and, with a
 *   window W >= 0, j >= pos0 + i - W) of sequence b.  Tokens before pos0 - W (the first query's
 *   window start) are never read: blocks holding only such tokens, and their table entries,
 *   may already have been released.
 * workspace: required, at least attn_prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D)
 *   bytes, 16-byte aligned, contents irrelevant: it receives contiguous copies of the visible
 *   key rows (with RoPE in the operand format of attn_rotate_keys_f16, bf16 without) and value
 *   rows.
 * Other arguments, the support matrix and the errors as in attn_prefill_chunk; also
 * ATTN_ERR_INVALID_ARG for a bad block size, a null or misaligned block table, or a chunk
 * past the table.  Table entries outside [0, num_blocks) are clamped into it.
 * --------------------------------------------------------------------------------------- */
size_t attn_prefill_chunk_paged_workspace_bytes(int B, int Hkv, int pos0, int Sq, int D);
attn_status attn_prefill_chunk_paged(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                     void* v_pages, int num_blocks, int block_size,
                                     const int32_t* block_table, int max_blocks, void* o, float* lse,
                                     attn_dtype out_dt, int B, int Hq, int Hkv, int Sq, int D, int pos0,
                                     int window, const float* rope_table, int table_max_pos,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_prefill_chunk_paged_varpos: attn_prefill_chunk_paged with a chunk start per sequence,
 * as attn_prefill_chunk_varpos does for a contiguous cache (same page sections): sequence b's
 * chunk goes to tokens p_b .. p_b+Sq-1, p_b = pos0[b], and its queries attend to its tokens
 * j <= p_b + i (and, with a window W >= 0, j >= p_b + i - W; tokens before p_b - W are never
 * read, so blocks holding only such tokens may already have been released).
 *
 * pos0: device int32 [B], 4-byte aligned, read on the device only; each value must lie in
 *   [0, pos0_max].  A sequence whose value lies outside gets NaN output rows (and NaN LSE),
 *   and none of its slots is written.
 * pos0_max: host int >= 0: pos0_max + Sq <= max_blocks * block_size, and with RoPE
 *   pos0_max + Sq <= table_max_pos.
 * workspace: required, at least attn_prefill_chunk_paged_workspace_bytes(B, Hkv, pos0_max, Sq, D)
 *   bytes, 16-byte aligned, contents irrelevant.
 * With every pos0[b] equal to p the result is attn_prefill_chunk_paged's with pos0 = p, bit for
 * bit.  Other arguments, layouts, the support matrix and the errors as in
 * attn_prefill_chunk_paged (with pos0_max in place of pos0); also ATTN_ERR_INVALID_ARG for a
 * null or misaligned pos0.
 * --------------------------------------------------------------------------------------- */
attn_status attn_prefill_chunk_paged_varpos(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                            void* v_pages, int num_blocks, int block_size,
                                            const int32_t* block_table, int max_blocks, const int32_t* pos0,
                                            int pos0_max, void* o, float* lse, attn_dtype out_dt, int B, int Hq,
                                            int Hkv, int Sq, int D, int window, const float* rope_table,
                                            int table_max_pos, void* workspace, size_t workspace_bytes,
                                            void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_cache_append, attn_cache_append_paged: write Sq new tokens of every sequence into a
 * KV cache and nothing else -- the step before attn_decode / attn_decode_paged in a serving loop
 * (ninaddeshpande.com, "The KV cache and the memory wall": each new token's key and value join
 * the cache, and the token then attends to the cache including itself).
 *
 * k_new, v_new: bf16 [B, Hkv, Sq, D] (k_new not yet rotated).  pos: device int32 [B], 4-byte
 * aligned: sequence b's tokens are written at positions pos[b] .. pos[b]+Sq-1; key row i is
 * RoPE(k_new row i) at position pos[b] + i, computed in float32 and rounded to bf16 (nearest
 * even), exactly as attn_prefill_chunk appends it; values are copied.  Nothing else is written.
 * attn_cache_append: k_cache, v_cache bf16 [B, Hkv, S_max, D], token t of sequence b in row t.
 * attn_cache_append_paged: the pools and block table of attn_decode_paged (token t of sequence
 *   b in block block_table[b * max_blocks + t / block_size], slot t % block_size; entries
 *   outside [0, num_blocks) are clamped into it).  The blocks receiving the tokens must not be
 *   shared between sequences.
 * A sequence whose pos[b] lies outside [0, cap - Sq] is not written, cap being the tokens the
 * cache holds (S_max, or max_blocks * block_size) and, with RoPE, at most table_max_pos.
 * rope_table: NULL stores the keys as given.  Errors: ATTN_ERR_INVALID_ARG for null pointers,
 * sizes < 1, Sq larger than the cache, misalignment, a bad block size, a table shorter than Sq;
 * ATTN_ERR_UNSUPPORTED for D outside {64, 128}.
 * --------------------------------------------------------------------------------------- */
attn_status attn_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* pos, int B, int Hkv, int Sq, int S_max, int D,
                              const float* rope_table, int table_max_pos, void* stream);
attn_status attn_cache_append_paged(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                                    int num_blocks, int block_size, const int32_t* block_table, int max_blocks,
                                    const int32_t* pos, int B, int Hkv, int Sq, int D, const float* rope_table,
                                    int table_max_pos, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_decode: one new query per sequence against a KV cache (ninaddeshpande.com, "The KV
 * cache and the memory wall"), split over the cache length ("split-K") with a merge pass.
 *
 * q: [B, Hq, 1, D] (not yet rotated); k_cache, v_cache: [B, Hkv, S_max, D], keys already
 * rotated (used exactly as stored); all of dtype in_dt.
 * cache_len, q_pos: device int32 [B].  Sequence b attends to cache rows
 * [0, min(cache_len[b], S_max)); its query is rotated at position q_pos[b] (if rope_table
 * is not NULL).  A row with cache_len[b] <= 0 yields o = 0 and lse = -inf.  A row whose
 * q_pos[b] lies outside [0, table_max_pos) yields NaN (the table has no such row).
 * Cache row j holds the token at position j; with a window W >= 0 only rows
 * j >= q_pos[b] - W are read and seen (q_pos is then required; a row with none left yields
 * o = 0 and lse = -inf).  Rows before the window are never used.
 * o: [B, Hq, 1, D] of dtype out_dt; lse: optional float32 [B, Hq].
 * n_split: number of cache chunks per (sequence, KV head); 0 picks one from the shape.
 * workspace: device scratch of at least attn_decode_workspace_bytes(...) bytes with the
 * same B, Hq, Hkv, S_max, D and n_split; its contents on entry do not matter.
 *
 * Support matrix: in_dt = ATTN_BF16, D in {64, 128}, out_dt either; any group size Hq / Hkv
 * (with more than 16 query heads per KV head, as in multi-query attention, a workgroup reads
 * each K/V tile once for up to 64 of them).
 * Errors: ATTN_ERR_INVALID_ARG for null pointers (q_pos may be NULL only without RoPE and
 * without a window), sizes < 1, Hq % Hkv != 0, n_split < 0, workspace too small, misalignment;
 * ATTN_ERR_UNSUPPORTED outside the support matrix.
 * --------------------------------------------------------------------------------------- */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int S_max, int D, int n_split);
int attn_decode_num_splits(int B, int Hq, int Hkv, int S_max, int D, int n_split);
attn_status attn_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cache_len, const int32_t* q_pos, void* o, float* lse,
                        attn_dtype in_dt, attn_dtype out_dt, int B, int Hq, int Hkv, int S_max,
                        int D, int window, const float* rope_table, int table_max_pos, int n_split,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_decode_noalloc: attn_decode for callers that cannot allocate device memory: code being
 * captured into a HIP graph, serving loops that must not allocate, harnesses that forbid it.
 *
 * Arguments, results and the support matrix are attn_decode's, without the workspace: the
 * partial results of the cache splits go to a buffer inside the library, a static device array
 * of ATTN_NOALLOC_SCRATCH_BYTES (16 MiB) on each GPU, created when the library's code object is
 * loaded on that GPU and held until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocator of any kind) and enqueues only kernel launches.  No part of the buffer needs to
 * start at zero: every partial the merge pass reads is written earlier in the same call.
 * Every call on one GPU uses that GPU's one buffer, so two calls that can overlap on the same GPU
 * (issued on different streams, or from different threads without ordering) race and corrupt
 * each other's results; the caller must order them.
 * Errors: those of attn_decode (except the workspace checks); ATTN_ERR_UNSUPPORTED when the
 * partials need more than the buffer holds, i.e. when attn_decode_workspace_bytes(B, Hq, Hkv,
 * S_max, D, n_split) > ATTN_NOALLOC_SCRATCH_BYTES (for example B = 32, Hq = 64, Hkv = 1,
 * 8192 keys needs 8.5 MB with the automatic split count); ATTN_ERR_HIP when the buffer's device
 * address cannot be obtained or the launch fails.
 * --------------------------------------------------------------------------------------- */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
attn_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* cache_len, const int32_t* q_pos, void* o, float* lse,
                                attn_dtype in_dt, attn_dtype out_dt, int B, int Hq, int Hkv, int S_max, int D,
                                int window, const float* rope_table, int table_max_pos, int n_split,
                                void* stream);

/* ---------------------------------------------------------------------------------------
 * attn_decode_paged: attn_decode against a paged KV cache.  The cache is a pool of
 * fixed-size physical blocks, allocated on demand and found through a per-sequence block
 * table like virtual-memory pages ("Building Self-Attention and Transformer Engines",
 * codingpancake.com, section 6.2; the page uses 16 tokens per block).
 *
 * k_pages, v_pages: [num_blocks, Hkv, block_size, D], keys already rotated (used as stored).
 * block_table: device int32 [B, max_blocks]; token t of sequence b is stored in block
 *   block_table[b * max_blocks + t / block_size], slot t % block_size.  Only the entries of
 *   blocks holding tokens [0, cache_len[b]) are read; the rest may hold anything.  An entry
 *   read outside [0, num_blocks) is clamped into it (no out-of-range access; the result is
 *   then meaningless).
 * cache_len, q_pos, q, o, lse, n_split, window, rope_table: as in attn_decode, with
 *   S_max = max_blocks * block_size (cache_len is clamped to it).  With a window, blocks that
 *   lie wholly before the window are not read (their table entries may be stale).
 * workspace: at least attn_decode_workspace_bytes(B, Hq, Hkv, max_blocks * block_size, D,
 *   n_split) bytes.
 * Support matrix: as attn_decode; block_size a power of two in [16, 4096].
 * Errors: ATTN_ERR_INVALID_ARG for null pointers, sizes < 1, a bad block_size, Hq % Hkv != 0,
 * workspace too small, misalignment; ATTN_ERR_UNSUPPORTED outside the support matrix.
 * --------------------------------------------------------------------------------------- */
attn_status attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, int num_blocks,
                              int block_size, const int32_t* block_table, int max_blocks,
                              const int32_t* cache_len, const int32_t* q_pos, void* o, float* lse,
                              attn_dtype in_dt, attn_dtype out_dt, int B, int Hq, int Hkv, int D,
                              int window, const float* rope_table, int table_max_pos, int n_split,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
