// Internal interface between the C ABI (mla_api.hip) and the kernels
// (mla_kernels.hip). Not installed; no HIP types beyond hipStream_t.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;         // tokens per page = keys per tile
constexpr int kDqk = 576;         // latent row: 512 latent + 64 rope
constexpr int kDv = 512;          // value = first 512 entries of the row
constexpr int kThreads = 256;     // 4 waves of 64 lanes per workgroup

// Metadata layout (int32 words, device):
//   [0] magic  [1] batch  [2] num_units  [3] units cut (U')  [4] total_partials
//   [5] units_used  [6] sequence start cost (tiles)
//   [7] max_pieces: the largest number of partials of one sequence
//   [8 .. 8+B]                 prefix: first flattened tile of each sequence [B+1]
//   [9+B .. 9+2B]              split_offset: first partial slot of each sequence [B+1]
//   [10+2B .. 10+2B+U)         unit_first_seq: sequence holding each unit's first tile
//   [10+2B+U .. 11+2B+2U)      unit_begin: first flattened tile of each unit [U+1]
//   [11+2B+2U .. 11+3B+2U)     seq_first_unit: unit holding each sequence's first tile
constexpr int kMdMagic = 0x4D4C4132;  // 'MLA2'
enum { MD_MAGIC = 0, MD_BATCH = 1, MD_UNITS = 2, MD_UNITS_CUT = 3, MD_TOTAL_PARTIALS = 4,
       MD_UNITS_USED = 5, MD_SEQ_COST = 6, MD_MAX_PIECES = 7, MD_HEADER = 8 };
constexpr int kDefaultMinTiles = 8;
// A sequence's start (query rows, epilogue, partial write, metadata) costs
// about as much as this many 64-token tiles; the split schedule charges it.
// Measured: ~1.4 tiles in the 16-row kernel, ~3.5 in the 64-row kernels.
constexpr int kSeqCostNarrow = 1;
constexpr int kSeqCostWide = 3;

inline size_t metadata_words(int batch, int units) {
  return (size_t)MD_HEADER + 3 * (size_t)batch + 2 + 2 * (size_t)units + 1;
}
__host__ __device__ inline size_t md_unit_begin(int batch, int units) { return (size_t)MD_HEADER + 2 * ((size_t)batch + 1) + units; }
__host__ __device__ inline size_t md_seq_first_unit(int batch, int units) { return md_unit_begin(batch, units) + units + 1; }

struct DecodeParams {
  const uint16_t* q;          // bf16 bits [B, s, H, 576], or [T, H, 576] with cu_q
  const uint8_t* kv;          // page pool bytes
  const float* kv_scale;      // [P, 64] (fp8 only)
  const int32_t* block_table; // [B, max_pages]
  const int32_t* seqlens;     // [B]
  const int32_t* cu_q;        // [B+1] query-token offsets (per-sequence q_len) or nullptr
  float* out;                 // [B, s, H, 512] or [T, H, 512]
  float* lse;                 // [B, s, H] or [T, H]
  const int32_t* md;          // metadata or nullptr (unsplit)
  float* ws_out;              // partial O  [slots, rows, 512]
  float* ws_lse;              // partial LSE [slots, rows]
  int batch, q_len, num_heads;
  int rows;                   // rows per sequence (q_len * H; the largest one with cu_q)
  int q_rows;                 // rows held by q (B * rows, or T * H with cu_q)
  int grid_units;             // work units of the launch (set by launch_decode)
  int max_pages;
  int num_pages;              // pages in the pool (page-id bounds checks of MLA_DEBUG_BOUNDS builds)
  float scale_log2;           // softmax_scale * log2(e)
};

// Kernel variants: rows of one workgroup and how its waves share a tile.
enum Variant {
  VAR_NARROW16 = 0,   // 16 rows; each wave takes 16 of the tile's 64 keys
  VAR_WIDE64X = 2,    // 64 rows; QK split 2x2 (rows x keys), PV split by columns
  VAR_Q8 = 3,         // 64 rows, fp8 cache on fp8 MFMA (queries and P quantised to E4M3)
};
int variant_for(int rows);
int variant_rows(int variant);

// ev_start / ev_stop: optional events recorded by the kernel dispatch itself.
hipError_t launch_decode(const DecodeParams& p, int variant, int grid_units, hipStream_t s,
                         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// 64-row kernel with score and output waves (mla_decode_so.hip), uniform q_len.
// fp8_mma: the fp8 cache on fp8 MFMA (queries and P in E4M3).
hipError_t launch_decode_so(const DecodeParams& p, int grid_units, hipStream_t s, hipEvent_t ev_start = nullptr,
                            hipEvent_t ev_stop = nullptr, bool fp8_mma = false);
hipError_t launch_metadata(const int32_t* seqlens, int batch, int units, int min_tiles, int seq_cost,
                           int32_t* md, hipStream_t s, hipEvent_t ev_start = nullptr,
                           hipEvent_t ev_stop = nullptr);
hipError_t launch_append(const uint16_t* latent, int batch, int new_tokens, const int32_t* block_table,
                         int max_pages, const int32_t* seqlens, uint8_t* kv, float* kv_scale, int fp8,
                         int num_pages, hipStream_t s);
// cu_q (nullable): per-sequence query offsets; sequence b then owns rows
// [0, (cu_q[b+1] - cu_q[b]) * num_heads) and writes out rows from cu_q[b] * num_heads.
// md (nullable): split metadata the offsets come from; nothing is merged
// unless its header names this batch and `units`.
hipError_t launch_combine(const float* part_out, const float* part_lse, const int32_t* offsets,
                          const int32_t* cu_q, int num_heads, int batch, int rows, float* out,
                          float* lse, int skip_single, hipStream_t s, const int32_t* md = nullptr,
                          int units = 0, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Device address of device `dev`'s static scratch (MLA_NOALLOC_SCRATCH_BYTES),
// looked up on the first call for that device, which must be current then.
hipError_t scratch_address(int dev, void** out);

// Prefill / extend (un-absorbed MLA, head dim 192 = 128 + 64 shared rope, v 128).
// Quantised prefill (mla_prefill_q8.hip): byte offsets of the quantised K,
// V, V scales and K scales inside one buffer, and its size.
struct QkvLayout {
  size_t k8, v8, vs, ks, bytes;
};
// total_k / 64 + batch tile slots per head; per (slot, head) record 12288
// bytes of K codes, 8192 of V codes, 256 E8M0 bytes and one fp32 K scale,
// each array starting 256-byte aligned.
inline QkvLayout qkv_layout(int batch, long long total_k, int num_heads) {
  auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t recs = (size_t)(total_k / 64 + batch) * (size_t)num_heads;
  QkvLayout l;
  l.k8 = 0;
  l.v8 = r256(recs * 12288);
  l.vs = l.v8 + r256(recs * 8192);
  l.ks = l.vs + r256(recs * 256);
  l.bytes = l.ks + r256(recs * sizeof(float));
  return l;
}
hipError_t launch_quant_kv(const uint16_t* k_nope, const uint16_t* k_rope, const uint16_t* v, const int32_t* cu_k,
                           int batch, long long total_k, int num_heads, uint8_t* qkv, hipStream_t s,
                           hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
int prefill_q8_rows_per_block();
hipError_t launch_prefill_q8(const uint16_t* q, const uint8_t* qkv, const int32_t* cu_q, const int32_t* cu_k,
                             int batch, int max_q_len, long long total_k, int num_heads, float softmax_scale,
                             float* out, float* lse, hipStream_t s, hipEvent_t ev_start = nullptr,
                             hipEvent_t ev_stop = nullptr);
// Page-id bounds violations counted by a MLA_DEBUG_BOUNDS build's decode
// kernels (one counter per translation unit); hipErrorNotSupported otherwise.
hipError_t page_violations_kernels(unsigned* count, bool reset);
hipError_t page_violations_so(unsigned* count, bool reset);
int prefill_rows_per_block();
hipError_t launch_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_rope, const uint16_t* v,
                          const int32_t* cu_q, const int32_t* cu_k, int batch, int max_q_len, int num_heads,
                          float softmax_scale, float* out, float* lse, hipStream_t s,
                          hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

}  // namespace mla
