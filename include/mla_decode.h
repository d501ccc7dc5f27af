/*
 * mla_decode.h -- C ABI of libmla_decode.so: Multi-head Latent Attention (MLA)
 * decode over a paged latent KV cache, hand-written HIP kernels for gfx950
 * (MI355X).
 *
 * What is computed (PaddleNLP issue #10157, "Multi-head Latent Attention (MLA)
 * operator", overview: one MLA pass is data load, QK GEMM, softmax update and
 * PV GEMM, adapted to decode with more than one token per request; its MTP
 * section: q_len > 1 verification at the original batch size):
 *
 *   for every sequence b, query token i < q_len, head h < num_heads:
 *     n      = clamp(L_b - q_len + i + 1, 0, L_b)      (causal rule)
 *     z_j    = softmax_scale * dot(q[b,i,h,0:576], K_j)     j < n
 *     out[b,i,h,:] = sum_j softmax(z)_j * V_j            V_j = K_j[0:512]
 *     lse[b,i,h]   = ln sum_j exp(z_j)                   (natural log)
 *   K_j is the 576-value latent row of token j (512 latent + 64 rope), shared
 *   by all heads; token j lives in page block_table[b][j / 64], slot j % 64.
 *   A row with n == 0 gets out = 0, lse = -inf.
 *   For the fp8 cache K_j = kv_scale[page][slot] * e4m3(code) (OCP E4M3FN).
 *
 * Conventions for every entry point:
 *   - Every pointer argument documented "device" is a device address on the
 *     current HIP device; the caller allocates, owns and frees all memory.
 *     The library allocates nothing and keeps no device state across calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it: no host synchronisation, no allocation.
 *   - Tensors are dense row-major (C order) with the shapes given.
 *   - Argument checking is host-side only (the library never reads device
 *     memory on the host). Checks run before any HIP call, so errors in
 *     arguments are reported even on a machine without a GPU.
 *   - Return value: an mla_status_t (as int). On failure mla_last_error()
 *     returns a thread-local message. Nothing is thrown or aborted across
 *     the ABI.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2
#define MLA_PAGE_TOKENS 64   /* tokens per cache page */
#define MLA_D_QK 576         /* query / latent row width: 512 latent + 64 rope */
#define MLA_D_V 512          /* value width: the first 512 entries of the row */
#define MLA_MAX_ROWS 4096    /* q_len * num_heads limit per sequence */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* NULL pointer, bad size, misaligned base pointer */
  MLA_ERR_UNSUPPORTED = 2,  /* dtype or device not supported (needs gfx950) */
  MLA_ERR_WORKSPACE = 3,    /* metadata or workspace buffer too small */
  MLA_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} mla_status_t;

typedef enum {
  MLA_KV_BF16 = 0,          /* cache holds bf16 values */
  MLA_KV_FP8_E4M3 = 1       /* cache holds OCP E4M3FN codes + fp32 per-token scale */
} mla_kv_dtype_t;

/* Library ABI version (MLA_ABI_VERSION of the build). */
int mla_abi_version(void);

/* Static string naming a status code. */
const char* mla_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* mla_last_error(void);

/*
 * Split-KV planning (host only, no device access).
 *
 * The split schedule cuts the flattened (sequence, 64-token tile) space into
 * `num_units` contiguous work units of about equal cost (FlashDecoding-style
 * splitting of the cache, named among the attention features in PaddleNLP
 * issue #10157's overview; the cache is cut into partitions that are merged
 * afterwards in the Append Attention flags of the mhpq.cn article on PaddleNLP
 * inference flags). A sequence's start (its query rows, its epilogue, its
 * metadata) is charged as c tiles: c = 1 when q_len * num_heads <= 16 (the
 * 16-row kernel), else c = 3 (the 64-row kernels). With T_b = ceil(L_b/64),
 * T = sum T_b, and every sequence with tiles laid on a weighted line as c
 * start positions then its T_b tiles (W positions in all):
 *   U' = max(1, min(num_units, floor(W / min_tiles_per_unit)))
 *   the line is cut at floor(u * W / U'), u = 0..U'; unit u < U' starts at
 *   the tile its cut names (a sequence's first tile if the cut falls in its
 *   start) and runs to the next unit's start; units u >= U' hold no tile.
 * A sequence touched by k > 1 units is computed as k partials and merged.
 *
 * mla_default_num_units: a unit count that fills the current device for this
 *   shape (0 if the device cannot be queried): 8 k for the 8 XCDs, with k the
 *   smallest multiple of c / gcd(c, rb) not below c / rb (c = CUs per XCD,
 *   rb = row blocks per sequence), so that the k rb workgroups an XCD runs
 *   fill whole rounds of its CUs.
 * mla_default_num_units_varlen: the same for mla_decode_fwd_varlen with up
 *   to max_q_len query tokens per sequence, with k also at least
 *   ceil(batch / 8) (about one unit per sequence: row blocks that sequences
 *   with fewer query tokens leave idle end their unit early and free their
 *   CU). Pass max_q_len as the q_len of mla_get_split_metadata.
 * mla_metadata_bytes: size of the metadata buffer for (batch, num_units).
 * mla_workspace_bytes: size of the partials workspace for the shape:
 *   (batch + num_units) * q_len * num_heads * (512 + 1) * 4 bytes, rounded up.
 */
int mla_default_num_units(int batch, int q_len, int num_heads);
int mla_default_num_units_varlen(int batch, int max_q_len, int num_heads);
size_t mla_metadata_bytes(int batch, int num_units);
size_t mla_workspace_bytes(int batch, int q_len, int num_heads, int num_units);

/*
 * mla_get_split_metadata: build the split schedule on the device.
 *   cache_seqlens  device int32 [batch], L_b >= 0 (negative values count as 0)
 *   batch          >= 1
 *   q_len, num_heads  >= 1, the shape of the decode calls that will use the
 *                  metadata (it selects the start cost c; any shape may still
 *                  use the metadata, only the balance differs)
 *   num_units      >= 1, the number of work units (see above)
 *   min_tiles_per_unit  >= 0; 0 selects the default (8)
 *   metadata       device buffer of >= mla_metadata_bytes(batch, num_units)
 *                  bytes, 4-byte aligned; fully written by this call
 *   stream         hipStream_t
 * One small kernel, stream-ordered. Reuse the metadata for every layer of a
 * decode step that has the same cache_seqlens.
 */
int mla_get_split_metadata(const int32_t* cache_seqlens, int batch, int q_len, int num_heads,
                           int num_units, int min_tiles_per_unit, void* metadata, size_t metadata_bytes,
                           void* stream);

/*
 * mla_decode_fwd: the decode attention (data load, QK GEMM, online softmax,
 * PV GEMM) and, when split, the LSE merge of the partials.
 *   q              device bf16 [batch, q_len, num_heads, 576], 16-byte aligned
 *   kv_cache       device [num_pages, 64, 576] of bf16 (MLA_KV_BF16) or E4M3FN
 *                  bytes (MLA_KV_FP8_E4M3), 16-byte aligned
 *   kv_scale       device fp32 [num_pages, 64], one scale per token; required
 *                  for MLA_KV_FP8_E4M3, ignored (may be NULL) for bf16
 *   kv_dtype       mla_kv_dtype_t
 *   num_pages      pages in the pool (>= 1)
 *   block_table    device int32 [batch, max_pages_per_seq]; entries
 *                  [0, ceil(L_b/64)) of row b must be valid page ids < num_pages.
 *                  The kernels may also load (and then ignore) other entries
 *                  of the table -- in split mode up to the first
 *                  min(64, max_pages_per_seq) of the row after a sequence's --
 *                  so the whole [batch, max_pages_per_seq] table must be
 *                  readable device memory; the values of entries past
 *                  ceil(L_b/64) never matter
 *   max_pages_per_seq  row stride of block_table (>= 1)
 *   cache_seqlens  device int32 [batch]; caller contract:
 *                  ceil(L_b/64) <= max_pages_per_seq
 *   batch, q_len, num_heads   >= 1; q_len * num_heads <= MLA_MAX_ROWS
 *   softmax_scale  finite
 *   out            device fp32 [batch, q_len, num_heads, 512], 16-byte aligned
 *   lse            device fp32 [batch, q_len, num_heads], 4-byte aligned
 *   metadata       NULL: one work unit per sequence, no partials, no merge
 *                  (workspace unused). Otherwise the buffer written by
 *                  mla_get_split_metadata for the same cache_seqlens, batch
 *                  and num_units (checked on the device against the buffer's
 *                  header: for another batch or num_units nothing is written).
 *   num_units      the value given to mla_get_split_metadata (ignored if
 *                  metadata is NULL)
 *   workspace      device buffer of >= mla_workspace_bytes(batch, q_len,
 *                  num_heads, num_units) bytes, 16-byte aligned (split only)
 *   stream         hipStream_t
 * Slots of a sequence's last page past L_b may hold any bytes (NaN included):
 * they never reach the outputs. Results are bitwise reproducible for a fixed
 * schedule (no atomics on the output path).
 */
int mla_decode_fwd(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                   int num_pages, const int32_t* block_table, int max_pages_per_seq,
                   const int32_t* cache_seqlens, int batch, int q_len, int num_heads,
                   float softmax_scale, float* out, float* lse,
                   const void* metadata, int num_units, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * mla_decode_fwd_fp8mma: mla_decode_fwd for an fp8 cache with both
 * contractions on fp8 matrix cores. PaddleNLP issue #10157 (quantization
 * section, SageAttention2) quantises P to FP8 and multiplies it with FP8 V,
 * dequantising the product once; this entry point does that and also
 * quantises the query rows:
 *   q8 = E4M3(q / sq) per row (round to nearest even) with sq = 2^k, k the
 *   smallest integer with max|q_row| <= 448 * 2^k (not below -126), so that
 *   q / sq is exact; scores from the E4M3 codes of q8 and the cache, times sq, the
 *   key's per-token scale and softmax_scale; P'_j = P_j * s_j (s_j the
 *   per-token scale) quantised to E4M3 per (row, 32-key block) with a
 *   power-of-two scale, undone exactly by the MFMA's block scale.
 * The result is an approximation of mla_decode_fwd's: on the normally
 * distributed test data the O error is a few percent of max|O| (the E4M3
 * rounding of q and P, relative 2^-4 per element) and the LSE error about
 * 0.03; the tests state the bound. Row sums and the LSE use unquantised P.
 *   kv_dtype       must be MLA_KV_FP8_E4M3 (else MLA_ERR_UNSUPPORTED)
 * Every other argument, the split plan, the workspace and the errors are
 * those of mla_decode_fwd; any q_len * num_heads <= MLA_MAX_ROWS works (rows
 * go in blocks of 64).
 */
int mla_decode_fwd_fp8mma(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                          int num_pages, const int32_t* block_table, int max_pages_per_seq,
                          const int32_t* cache_seqlens, int batch, int q_len, int num_heads,
                          float softmax_scale, float* out, float* lse, const void* metadata, int num_units,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_fwd_varlen: mla_decode_fwd with a query count per sequence, so
 * one forward verifies sequences that accepted different numbers of draft
 * tokens in the previous round (PaddleNLP issue #10157, MTP section: the
 * verification pass keeps the batch and handles each request's 1 + drafts
 * tokens; q_len up to 6 there).
 *   q              device bf16 bits [total_q, num_heads, 576], 16-byte aligned;
 *                  the s_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] query tokens
 *                  of sequence b are rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]
 *   cu_seqlens_q   device int32 [batch + 1], cu[0] = 0, non-decreasing,
 *                  cu[batch] <= total_q, every s_b <= max_q_len (caller
 *                  contract: the library does not read it on the host)
 *   total_q        rows of q (>= 1); max_q_len >= 1, max_q_len * num_heads <= MLA_MAX_ROWS
 *   out, lse       device fp32 [total_q, num_heads, 512] / [total_q, num_heads];
 *                  rows of sequences with s_b = 0 and rows past cu[batch] are
 *                  not written
 * Causal rule per sequence: query i < s_b sees keys j <= L_b - s_b + i.
 * metadata / workspace: from mla_get_split_metadata and
 * mla_workspace_bytes(batch, max_q_len, num_heads, num_units), as for
 * mla_decode_fwd. All other arguments, errors and guarantees are those of
 * mla_decode_fwd.
 */
int mla_decode_fwd_varlen(const void* q, const int32_t* cu_seqlens_q, int total_q, int max_q_len,
                          const void* kv_cache, const float* kv_scale, int kv_dtype, int num_pages,
                          const int32_t* block_table, int max_pages_per_seq, const int32_t* cache_seqlens,
                          int batch, int num_heads, float softmax_scale, float* out, float* lse,
                          const void* metadata, int num_units, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * mla_prefill_fwd: the second workload, prefill / extend attention in the
 * un-absorbed MLA form. Per head the key is [k_nope_h, k_rope] (head dim 192
 * = 128 + 64, the DeepSeek head dim PaddleNLP issue #10157 gives for its long
 * prefill attention, quantization section, SageAttention; the rope part is
 * shared by all heads) and the value is v_h (128). Sequence b's N_b new
 * tokens are the last N_b of its L_b tokens (prefill: N_b = L_b; extend: a
 * cached prefix of L_b - N_b tokens); query i sees keys j <= L_b - N_b + i.
 *   q              device bf16 bits [total_q, num_heads, 192], 16-byte aligned
 *   k_nope         device bf16 bits [total_k, num_heads, 128], 16-byte aligned
 *   k_rope         device bf16 bits [total_k, 64], 16-byte aligned
 *   v              device bf16 bits [total_k, num_heads, 128], 16-byte aligned
 *   cu_seqlens_q   device int32 [batch + 1]: sequence b owns q rows
 *                  cu_q[b] .. cu_q[b+1] (N_b <= max_q_len)
 *   cu_seqlens_k   device int32 [batch + 1]: sequence b owns key rows
 *                  cu_k[b] .. cu_k[b+1] (L_b >= N_b; caller contract, not
 *                  read on the host)
 *   batch, max_q_len, num_heads   >= 1; num_heads <= 65535
 *   softmax_scale  finite (1/sqrt(192) for DeepSeek)
 *   out            device fp32 [total_q, num_heads, 128], 16-byte aligned
 *   lse            device fp32 [total_q, num_heads] (natural log)
 *   stream         hipStream_t or NULL
 * Rows of sequences with N_b = 0 are not written. The library allocates
 * nothing. Errors: MLA_ERR_INVALID_ARG for NULL or misaligned pointers and
 * out-of-range sizes, MLA_ERR_HIP for a failed launch.
 */
int mla_prefill_fwd(const void* q, const void* k_nope, const void* k_rope, const void* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int max_q_len,
                    int num_heads, float softmax_scale, float* out, float* lse, void* stream);

/*
 * Quantised prefill / extend: the dynamic quantisation of PaddleNLP issue
 * #10157's quantization section (SageAttention, DeepSeek head dim 192) --
 * Q and K quantised to INT8, V to FP8; the INT32 products Q.K^T turned into
 * FP32 and dequantised, an online softmax over them, its P quantised to FP8
 * and multiplied with the FP8 V, the product dequantised once. Same inputs,
 * outputs and causal rule as mla_prefill_fwd. The pages fix no block sizes or
 * scale rules; this library's:
 *   Q: INT8 per (query token, head): scale = max|q| / 127 over the 192
 *      features (fp32), code = clamp(rint(q * (127 / max|q|)), +-127);
 *   K: INT8 per (sequence, 64-key tile counted from the sequence's first key,
 *      head), the same rule over the tile's valid keys x 192 features
 *      (features 0-127: the head's k_nope, 128-191: k_rope);
 *   V: E4M3FN per (sequence, 32-key block, head, feature) with the scale
 *      2^e, e the smallest integer with max|v| <= 448 * 2^e (clamped to
 *      [-127, 127]; 0 for an all-zero block), code = nearest-even E4M3FN of
 *      v * 2^-e (exact);
 *   P: the online softmax raises its running max to every 64-key tile's max
 *      (so P <= 1) and quantises P * 2^8 to E4M3FN; the row sum adds the
 *      unquantised P.
 * A row with no visible key gets O = 0, LSE = -inf.
 *
 * mla_prefill_quant_kv_bytes: size of the quantised K/V buffer ("qkv") for
 *   total_k keys (= cu_seqlens_k[batch]); 0 for invalid sizes. Host-only.
 *   Layout (for tests and tools; n = total_k / 64 + batch tile slots, the
 *   tile t of sequence b in slot T = cu_k[b] / 64 + b + t, record R = T * H + h):
 *     k8 at 0: 12288 bytes per record; byte f*1024 + l*16 + i is the INT8
 *        code of K[key 64t + 32(f/6) + l%32][feature 32(f%6) + 16(l/32) + i];
 *     v8 at round256(n*H*12288): 8192 bytes per record; byte
 *        (2g + q)*1024 + l*16 + i is the E4M3FN code of V[key 64t + 32q +
 *        8(i/4) + 4(l/32) + i%4][feature 32g + l%32];
 *     vs after v8 (each array starts 256-aligned): 256 bytes per record; byte
 *        4l + g = 127 + e of (feature 32g + l%32, 32-key block 2t + l/32);
 *     ks after vs: one fp32 K scale per record.
 *   Keys past the sequence end hold code 0; slots between sequences are not
 *   written.
 * mla_prefill_quantize_kv: fills qkv from the bf16 k_nope [total_k, H, 128],
 *   k_rope [total_k, 64], v [total_k, H, 128] (16-byte aligned) and
 *   cu_seqlens_k [batch + 1] (non-decreasing, cu_k[batch] = total_k: caller
 *   contract, not read on the host). qkv: device, 256-byte aligned,
 *   >= mla_prefill_quant_kv_bytes bytes, else MLA_ERR_WORKSPACE.
 * mla_prefill_quant_fwd: attention of q [total_q, H, 192] bf16 (quantised
 *   in the kernel) over a qkv filled by mla_prefill_quantize_kv for the same
 *   cu_seqlens_k, batch, total_k and num_heads; out [total_q, H, 128] fp32,
 *   lse [total_q, H] (natural log); rows of sequences with N_b = 0 are not
 *   written. The library allocates nothing. Errors: MLA_ERR_INVALID_ARG for
 *   NULL or misaligned pointers and out-of-range sizes (num_heads <= 65535),
 *   MLA_ERR_WORKSPACE for a short qkv, MLA_ERR_HIP for a failed launch.
 */
size_t mla_prefill_quant_kv_bytes(int batch, int64_t total_k, int num_heads);
int mla_prefill_quantize_kv(const void* k_nope, const void* k_rope, const void* v, const int32_t* cu_seqlens_k,
                            int batch, int64_t total_k, int num_heads, void* qkv, size_t qkv_bytes, void* stream);
int mla_prefill_quant_fwd(const void* q, const void* qkv, size_t qkv_bytes, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int batch, int max_q_len, int64_t total_k, int num_heads,
                          float softmax_scale, float* out, float* lse, void* stream);

/*
 * mla_combine: merge per-sequence partials by their log-sum-exp, the merge
 * step of split-KV decoding (FlashDecoding, named among the attention
 * features in PaddleNLP issue #10157's overview; the cache partitions of
 * Append Attention that are computed apart and merged, mhpq.cn article on
 * PaddleNLP inference flags, Append Attention section). Partials of disjoint
 * key sets combine exactly: each is renormalised by exp(lse_k - lse) of the
 * softmax over their union.
 *   part_out        device fp32 [num_partials, rows_per_seq, 512], 16-byte aligned
 *   part_lse        device fp32 [num_partials, rows_per_seq] (natural log)
 *   seq_part_offsets device int32 [batch + 1], non-decreasing; sequence b owns
 *                   partials [off[b], off[b+1])
 *   batch, rows_per_seq  >= 1; rows_per_seq <= MLA_MAX_ROWS
 *   out             device fp32 [batch, rows_per_seq, 512], 16-byte aligned
 *   lse             device fp32 [batch, rows_per_seq]
 * Per row: M = max_k lse_k; lse = M + ln sum_k exp(lse_k - M);
 * out = sum_k exp(lse_k - lse) * part_out_k. Partials with lse_k = -inf weigh
 * 0 and their part_out values are not read into the result (NaN included); a
 * sequence with no partial (or only -inf ones) gets out = 0, lse = -inf.
 */
int mla_combine(const float* part_out, const float* part_lse, const int32_t* seq_part_offsets,
                int batch, int rows_per_seq, float* out, float* lse, void* stream);

/*
 * mla_append_kv: store each sequence's newest latent rows in their cache
 * pages -- the step just before attention in a decode step. The 8-bit cache
 * is the C8 precision among the cache precisions listed in PaddleNLP issue
 * #10157's overview, stored here as OCP E4M3FN codes with one fp32 scale per
 * token.
 *   latent         device bf16 bits [batch, new_tokens, 576], 16-byte aligned
 *   batch, new_tokens   >= 1
 *   block_table    device int32 [batch, max_pages_per_seq]
 *   cache_seqlens  device int32 [batch]: lengths that already INCLUDE the new
 *                  tokens (the same array the following mla_decode_fwd uses).
 *                  Token i of sequence b is position j = L_b - new_tokens + i,
 *                  stored at page block_table[b][j / 64], slot j % 64.
 *                  Positions j < 0, j / 64 >= max_pages_per_seq, or page ids
 *                  outside [0, num_pages) are skipped (nothing is written).
 *   kv_cache       device [num_pages, 64, 576] bf16 or E4M3FN codes; written
 *                  only at the appended (page, slot) rows; 16-byte aligned
 *   kv_scale       device fp32 [num_pages, 64] (fp8 only; NULL for bf16);
 *                  written only at the appended rows
 *   kv_dtype       mla_kv_dtype_t
 * bf16: the row's bits are copied. fp8: scale = max_d |x_d| / 448 (1 for an
 * all-zero row) and code_d = nearest-even E4M3FN of clamp(x_d / scale, -448,
 * 448), every step one correctly rounded fp32 operation. Rows with
 * non-finite values are not supported. Two calls that append to the same
 * (page, slot) race; different sequences must not share appended positions.
 */
int mla_append_kv(const void* latent, int batch, int new_tokens, const int32_t* block_table,
                  int max_pages_per_seq, const int32_t* cache_seqlens, void* kv_cache, float* kv_scale,
                  int kv_dtype, int num_pages, void* stream);

/*
 * mla_decode_fwd_noalloc: mla_decode_fwd for callers that cannot allocate
 * device memory -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. One call builds the split schedule and
 * runs the split decode and the merge, with the schedule and the partials in
 * a static device buffer of MLA_NOALLOC_SCRATCH_BYTES that the library holds
 * on each device it runs on until the process ends (its device address is
 * looked up once per device on the first call there). The call allocates
 * nothing and takes no workspace.
 *   num_units      >= 0; 0 selects mla_default_num_units(batch, q_len, num_heads)
 *   min_tiles_per_unit  >= 0; 0 selects the default (8)
 *   every other argument as for mla_decode_fwd.
 * Limit: mla_noalloc_scratch_need(batch, q_len, num_heads, units) must not
 * exceed MLA_NOALLOC_SCRATCH_BYTES (metadata rounded up to 256 bytes plus
 * mla_workspace_bytes for the shape); larger calls fail with
 * MLA_ERR_WORKSPACE before anything is launched.
 * All calls on one device share its buffer: calls that overlap in time on
 * that device (other streams, other threads) race and must be serialised by
 * the caller. Nothing in the buffer needs clearing between calls: every word
 * a call reads was written earlier by the same call. Results equal
 * mla_decode_fwd's with a plan of the same unit count, bit for bit.
 * mla_noalloc_scratch_need: the bytes a call of this shape uses (0 for
 * invalid sizes).
 */
#define MLA_NOALLOC_SCRATCH_BYTES (128u << 20)
size_t mla_noalloc_scratch_need(int batch, int q_len, int num_heads, int num_units);
int mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                           int num_pages, const int32_t* block_table, int max_pages_per_seq,
                           const int32_t* cache_seqlens, int batch, int q_len, int num_heads,
                           float softmax_scale, float* out, float* lse, int num_units, int min_tiles_per_unit,
                           void* stream);

/*
 * mla_debug_page_violations: page-id bounds checks (diagnostics). The decode
 * entry points trust block_table (caller contract above). A library built
 * with MLA_DEBUG_BOUNDS (libmla_decode_debug.so) checks every page id its
 * decode kernels use against [0, num_pages): an id outside is counted and
 * replaced by page 0, so no read leaves the pool (the result is then not
 * meaningful). This call waits for the device, returns the number of
 * violations counted since the last reset in *count (per page use, summed
 * over the kernels), and clears the counters when reset != 0. Without
 * MLA_DEBUG_BOUNDS it returns MLA_ERR_UNSUPPORTED.
 */
int mla_debug_page_violations(int reset, uint64_t* count);

/*
 * Measurement hook (diagnostics, not part of the computation).
 * mla_profile_enable(1): from now on every kernel launch of the library is
 *   bracketed by a pair of HIP events recorded by the dispatch itself on the
 *   caller's stream, so each interval is that kernel's execution (no launch
 *   latency). Launches are recorded per kind:
 *     MLA_PROFILE_ATTENTION  the attention kernel of mla_decode_fwd and its
 *                            variants, and the kernels of mla_prefill_fwd and
 *                            mla_prefill_quant_fwd
 *     MLA_PROFILE_METADATA   the kernel of mla_get_split_metadata
 *     MLA_PROFILE_COMBINE    the LSE merge (of a split decode or mla_combine)
 *     MLA_PROFILE_QUANTIZE   the K/V quantiser of mla_prefill_quantize_kv
 *   Event pairs come from a pool the library creates on first use (host-side
 *   HIP event objects; no device memory). mla_profile_enable(0) stops
 *   recording.
 * mla_profile_read_launches: waits for the recorded events of one kind, writes
 *   the elapsed time (ms) of each recorded launch in launch order to
 *   ms[0 .. min(count, capacity)), sets *count to the number recorded, and
 *   clears that kind's record. capacity may be 0 (ms may then be NULL).
 * mla_profile_read: the same for MLA_PROFILE_ATTENTION, as the summed time.
 * Not thread-safe with concurrent decode calls on other threads.
 */
#define MLA_PROFILE_ATTENTION 0
#define MLA_PROFILE_METADATA 1
#define MLA_PROFILE_COMBINE 2
#define MLA_PROFILE_QUANTIZE 3
int mla_profile_enable(int enable);
int mla_profile_read_launches(int kernel, float* ms, int capacity, int* count);
int mla_profile_read(double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
