// C ABI of libmla_decode.so (declared in include/mla_decode.h): host-side
// argument checks, split planning and kernel launches. No device memory is
// read or allocated here.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "mla_decode.h"
#include "mla_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Device facts, queried once per device.
struct DevInfo {
  int checked = 0;
  int supported = 0;
  int cus = 0;
  char arch[64] = "";
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

int device_info(DevInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MLA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    strncpy(d.arch, prop.gcnArchName, sizeof(d.arch) - 1);
    d.supported = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.checked = 1;
  }
  *out = d;
  if (!d.supported) return fail(MLA_ERR_UNSUPPORTED, "device arch %s is not gfx950", d.arch);
  return MLA_OK;
}

// Measurement hook state (see mla_profile_enable): per kernel kind, the
// (start, stop) event pairs recorded by the dispatches, in launch order.
constexpr int kProfKinds = 4;   // MLA_PROFILE_ATTENTION, _METADATA, _COMBINE, _QUANTIZE
struct Profile {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;                                         // free events
  std::vector<std::pair<hipEvent_t, hipEvent_t>> recorded[kProfKinds];  // (start, stop)
};
Profile g_prof;

hipEvent_t take_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// An event pair for the next launch when recording is on (else nulls).
void prof_begin(hipEvent_t* ev0, hipEvent_t* ev1) {
  *ev0 = *ev1 = nullptr;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.on) return;
  *ev0 = take_event();
  *ev1 = take_event();
  if (!*ev0 || !*ev1) {
    if (*ev0) g_prof.pool.push_back(*ev0);
    if (*ev1) g_prof.pool.push_back(*ev1);
    *ev0 = *ev1 = nullptr;
  }
}

// Keep the pair of a launch that was made (return it to the pool otherwise).
void prof_end(int kind, hipEvent_t ev0, hipEvent_t ev1, bool launched) {
  if (!ev0 || !ev1) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (launched) {
    g_prof.recorded[kind].emplace_back(ev0, ev1);
  } else {
    g_prof.pool.push_back(ev0);
    g_prof.pool.push_back(ev1);
  }
}

size_t workspace_need(int batch, int q_len, int num_heads, int units) {
  const size_t slots = (size_t)batch + (size_t)units;
  const size_t rows = (size_t)q_len * (size_t)num_heads;
  const size_t o_bytes = slots * rows * mla::kDv * sizeof(float);
  const size_t l_bytes = slots * rows * sizeof(float);
  return o_bytes + ((l_bytes + 255) & ~(size_t)255);
}


// One 147 KiB-LDS workgroup per CU. Workgroups are dealt to the 8 XCDs round
// robin, and the rb row blocks of a unit share one XCD (they read the same
// pages through its L2), so an XCD runs k units as k * rb workgroups on its
// CUs. k is the smallest multiple of per_xcd / gcd(per_xcd, rb) that is at
// least max(per_xcd / rb, k_floor, 1): k * rb then fills whole rounds of the
// XCD's CUs, never leaving a second round a few workgroups deep (e.g. rb =
// 12: k = 8, three full rounds, where k = 2 or 3 would leave 8 CUs idle or
// run 4 workgroups in a second round). Returns 8k, or 0 on a device error.
int units_in_whole_rounds(int batch, int q_len, int num_heads, int k_floor) {
  if (batch < 1 || q_len < 1 || num_heads < 1) return 0;
  DevInfo d;
  if (device_info(&d) != MLA_OK) return 0;
  const int rows = q_len * num_heads;
  const int var = mla::variant_for(rows);
  const int rb = (rows + mla::variant_rows(var) - 1) / mla::variant_rows(var);
  constexpr int kXcds = 8;
  const int per_xcd = d.cus / kXcds > 0 ? d.cus / kXcds : 1;
  int g = per_xcd, r = rb;
  while (r) { const int t = g % r; g = r; r = t; }
  const int step = per_xcd / g;
  int k0 = per_xcd / rb;
  if (k0 < k_floor) k0 = k_floor;
  if (k0 < 1) k0 = 1;
  const int k = ((k0 + step - 1) / step) * step;
  return k * kXcds;
}
}  // namespace

extern "C" {

int mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return g_err; }


int mla_default_num_units(int batch, int q_len, int num_heads) {
  return units_in_whole_rounds(batch, q_len, num_heads, 0);
}

int mla_default_num_units_varlen(int batch, int max_q_len, int num_heads) {
  // about one unit per sequence: the row blocks that a sequence with fewer
  // query tokens leaves idle then end their unit early and free their CU for
  // the next workgroup, instead of idling beside a longer neighbour
  return units_in_whole_rounds(batch, max_q_len, num_heads, (batch + 7) / 8);
}

size_t mla_metadata_bytes(int batch, int num_units) {
  if (batch < 1 || num_units < 1) return 0;
  return mla::metadata_words(batch, num_units) * sizeof(int32_t);
}

size_t mla_workspace_bytes(int batch, int q_len, int num_heads, int num_units) {
  if (batch < 1 || q_len < 1 || num_heads < 1 || num_units < 1) return 0;
  return workspace_need(batch, q_len, num_heads, num_units);
}

int mla_get_split_metadata(const int32_t* cache_seqlens, int batch, int q_len, int num_heads,
                           int num_units, int min_tiles_per_unit, void* metadata, size_t metadata_bytes,
                           void* stream) {
  if (!cache_seqlens || !metadata) return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  if (q_len < 1 || num_heads < 1)
    return fail(MLA_ERR_INVALID_ARG, "q_len and num_heads must be >= 1 (got %d, %d)", q_len, num_heads);
  if (num_units < 1) return fail(MLA_ERR_INVALID_ARG, "num_units must be >= 1 (got %d)", num_units);
  if (min_tiles_per_unit < 0)
    return fail(MLA_ERR_INVALID_ARG, "min_tiles_per_unit must be >= 0 (got %d)", min_tiles_per_unit);
  if (!aligned(cache_seqlens, 4) || !aligned(metadata, 4))
    return fail(MLA_ERR_INVALID_ARG, "cache_seqlens and metadata must be 4-byte aligned");
  if (metadata_bytes < mla_metadata_bytes(batch, num_units))
    return fail(MLA_ERR_WORKSPACE, "metadata buffer has %zu bytes, needs %zu", metadata_bytes,
                mla_metadata_bytes(batch, num_units));
  DevInfo d;
  int st = device_info(&d);
  if (st != MLA_OK) return st;
  const int mt = min_tiles_per_unit == 0 ? mla::kDefaultMinTiles : min_tiles_per_unit;
  // a sequence's start costs what it does in the kernel this shape selects
  const int rows = q_len * num_heads;
  const int cost = mla::variant_for(rows) == mla::VAR_NARROW16 ? mla::kSeqCostNarrow : mla::kSeqCostWide;
  hipEvent_t ev0, ev1;
  prof_begin(&ev0, &ev1);
  hipError_t e = mla::launch_metadata(cache_seqlens, batch, num_units, mt, cost, (int32_t*)metadata,
                                      (hipStream_t)stream, ev0, ev1);
  prof_end(MLA_PROFILE_METADATA, ev0, ev1, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "metadata kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Split-schedule build that decode_impl launches itself, after its argument
// checks (mla_decode_fwd_noalloc).
struct MetadataLaunch {
  int min_tiles;
  int seq_cost;
};

// Shared body of mla_decode_fwd (cu_q == nullptr: q_len query tokens per
// sequence) and mla_decode_fwd_varlen (cu_q: per-sequence offsets, q_len is
// the largest count, q holds total_q tokens).
int decode_impl(const void* q, const int32_t* cu_q, int total_q, const void* kv_cache, const float* kv_scale,
                int kv_dtype, int num_pages, const int32_t* block_table, int max_pages_per_seq,
                const int32_t* cache_seqlens, int batch, int q_len, int num_heads, float softmax_scale,
                float* out, float* lse, const void* metadata, int num_units, void* workspace,
                size_t workspace_bytes, void* stream, bool fp8_mma = false,
                const MetadataLaunch* build_metadata = nullptr) {
  if (!q || !kv_cache || !block_table || !cache_seqlens || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (fp8_mma && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "the fp8-MFMA path needs an fp8 cache (kv_dtype %d)", kv_dtype);
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "kv_dtype %d is not supported", kv_dtype);
  if (kv_dtype == MLA_KV_FP8_E4M3 && !kv_scale)
    return fail(MLA_ERR_INVALID_ARG, "fp8 cache needs kv_scale");
  if (batch < 1 || q_len < 1 || num_heads < 1)
    return fail(MLA_ERR_INVALID_ARG, "batch, q_len, num_heads must be >= 1 (got %d, %d, %d)", batch,
                q_len, num_heads);
  if ((long long)q_len * num_heads > MLA_MAX_ROWS)
    return fail(MLA_ERR_INVALID_ARG, "q_len * num_heads = %lld exceeds %d", (long long)q_len * num_heads,
                MLA_MAX_ROWS);
  if (cu_q && total_q < 1) return fail(MLA_ERR_INVALID_ARG, "total_q must be >= 1");
  if ((long long)(cu_q ? total_q : (long long)batch * q_len) * num_heads > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARG, "query rows exceed the 32-bit row index");
  if (num_pages < 1 || max_pages_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARG, "num_pages and max_pages_per_seq must be >= 1");
  if (!isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16))
    return fail(MLA_ERR_INVALID_ARG, "q, kv_cache and out must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(block_table, 4) || !aligned(cache_seqlens, 4) ||
      (kv_scale && !aligned(kv_scale, 4)) || (cu_q && !aligned(cu_q, 4)))
    return fail(MLA_ERR_INVALID_ARG, "lse, block_table, cache_seqlens, kv_scale, cu_seqlens_q must be 4-byte aligned");
  if (metadata) {
    if (num_units < 1) return fail(MLA_ERR_INVALID_ARG, "num_units must be >= 1 with metadata");
    if ((long long)batch * q_len * num_heads > INT32_MAX)
      return fail(MLA_ERR_INVALID_ARG, "batch * q_len * num_heads exceeds the merge's 32-bit row index");
    if (!aligned(metadata, 4)) return fail(MLA_ERR_INVALID_ARG, "metadata must be 4-byte aligned");
    if (!workspace || !aligned(workspace, 16))
      return fail(MLA_ERR_INVALID_ARG, "split decode needs a 16-byte aligned workspace");
    const size_t need = workspace_need(batch, q_len, num_heads, num_units);
    if (workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  DevInfo d;
  int st = device_info(&d);
  if (st != MLA_OK) return st;

  mla::DecodeParams p;
  p.q = (const uint16_t*)q;
  p.kv = (const uint8_t*)kv_cache;
  p.kv_scale = kv_dtype == MLA_KV_FP8_E4M3 ? kv_scale : nullptr;   // selects the fp8 kernels
  p.block_table = block_table;
  p.seqlens = cache_seqlens;
  p.cu_q = cu_q;
  p.out = out;
  p.lse = lse;
  p.md = (const int32_t*)metadata;
  p.batch = batch;
  p.q_len = q_len;
  p.num_heads = num_heads;
  p.rows = q_len * num_heads;
  p.q_rows = cu_q ? total_q * num_heads : batch * p.rows;
  p.max_pages = max_pages_per_seq;
  p.num_pages = num_pages;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  const size_t slots = (size_t)batch + (size_t)num_units;
  p.ws_out = metadata ? (float*)workspace : nullptr;
  p.ws_lse = metadata ? (float*)((char*)workspace + slots * p.rows * mla::kDv * sizeof(float)) : nullptr;

  const int var = fp8_mma ? mla::VAR_Q8 : mla::variant_for(p.rows);
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t ev0, ev1;
  if (build_metadata) {
    // the schedule into `metadata`, stream-ordered before the attention kernel
    prof_begin(&ev0, &ev1);
    hipError_t e = mla::launch_metadata(cache_seqlens, batch, num_units, build_metadata->min_tiles,
                                        build_metadata->seq_cost, (int32_t*)metadata, s, ev0, ev1);
    prof_end(MLA_PROFILE_METADATA, ev0, ev1, e == hipSuccess);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "metadata kernel launch: %s", hipGetErrorString(e));
  }
  prof_begin(&ev0, &ev1);
  hipError_t e = mla::launch_decode(p, var, metadata ? num_units : batch, s, ev0, ev1);
  prof_end(MLA_PROFILE_ATTENTION, ev0, ev1, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode kernel launch: %s", hipGetErrorString(e));
  if (metadata) {
    const int32_t* offsets = (const int32_t*)metadata + mla::MD_HEADER + batch + 1;
    prof_begin(&ev0, &ev1);
    e = mla::launch_combine(p.ws_out, p.ws_lse, offsets, cu_q, num_heads, batch, p.rows, out, lse, 1, s,
                            p.md, num_units, ev0, ev1);
    prof_end(MLA_PROFILE_COMBINE, ev0, ev1, e == hipSuccess);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

int mla_decode_fwd(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                   int num_pages, const int32_t* block_table, int max_pages_per_seq,
                   const int32_t* cache_seqlens, int batch, int q_len, int num_heads,
                   float softmax_scale, float* out, float* lse, const void* metadata, int num_units,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, nullptr, 0, kv_cache, kv_scale, kv_dtype, num_pages, block_table, max_pages_per_seq,
                     cache_seqlens, batch, q_len, num_heads, softmax_scale, out, lse, metadata, num_units,
                     workspace, workspace_bytes, stream);
}

int mla_decode_fwd_fp8mma(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                          int num_pages, const int32_t* block_table, int max_pages_per_seq,
                          const int32_t* cache_seqlens, int batch, int q_len, int num_heads,
                          float softmax_scale, float* out, float* lse, const void* metadata, int num_units,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, nullptr, 0, kv_cache, kv_scale, kv_dtype, num_pages, block_table, max_pages_per_seq,
                     cache_seqlens, batch, q_len, num_heads, softmax_scale, out, lse, metadata, num_units,
                     workspace, workspace_bytes, stream, true);
}

int mla_decode_fwd_varlen(const void* q, const int32_t* cu_seqlens_q, int total_q, int max_q_len,
                          const void* kv_cache, const float* kv_scale, int kv_dtype, int num_pages,
                          const int32_t* block_table, int max_pages_per_seq, const int32_t* cache_seqlens,
                          int batch, int num_heads, float softmax_scale, float* out, float* lse,
                          const void* metadata, int num_units, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!cu_seqlens_q) return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  return decode_impl(q, cu_seqlens_q, total_q, kv_cache, kv_scale, kv_dtype, num_pages, block_table,
                     max_pages_per_seq, cache_seqlens, batch, max_q_len, num_heads, softmax_scale, out, lse,
                     metadata, num_units, workspace, workspace_bytes, stream);
}

int mla_prefill_fwd(const void* q, const void* k_nope, const void* k_rope, const void* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int max_q_len,
                    int num_heads, float softmax_scale, float* out, float* lse, void* stream) {
  if (!q || !k_nope || !k_rope || !v || !cu_seqlens_q || !cu_seqlens_k || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (batch < 1 || max_q_len < 1 || num_heads < 1)
    return fail(MLA_ERR_INVALID_ARG, "batch, max_q_len, num_heads must be >= 1 (got %d, %d, %d)", batch,
                max_q_len, num_heads);
  if (num_heads > 65535) return fail(MLA_ERR_INVALID_ARG, "num_heads must be <= 65535");
  const long long nblk = ((long long)max_q_len + mla::prefill_rows_per_block() - 1) / mla::prefill_rows_per_block();
  // the kernel's linear workgroup id runs over (query block, sequence, head) in an int
  if (nblk * batch * num_heads > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARG, "batch * query blocks * num_heads exceeds the 32-bit grid index");
  if (!isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (!aligned(q, 16) || !aligned(k_nope, 16) || !aligned(k_rope, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(MLA_ERR_INVALID_ARG, "q, k_nope, k_rope, v and out must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return fail(MLA_ERR_INVALID_ARG, "lse and the offsets must be 4-byte aligned");
  DevInfo d;
  int st = device_info(&d);
  if (st != MLA_OK) return st;
  hipEvent_t ev0, ev1;
  prof_begin(&ev0, &ev1);
  hipError_t e = mla::launch_prefill((const uint16_t*)q, (const uint16_t*)k_nope, (const uint16_t*)k_rope,
                                     (const uint16_t*)v, cu_seqlens_q, cu_seqlens_k, batch, max_q_len, num_heads,
                                     softmax_scale, out, lse, (hipStream_t)stream, ev0, ev1);
  prof_end(MLA_PROFILE_ATTENTION, ev0, ev1, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(e));
  return ok();
}

size_t mla_prefill_quant_kv_bytes(int batch, int64_t total_k, int num_heads) {
  if (batch < 1 || total_k < 0 || num_heads < 1) return 0;
  return mla::qkv_layout(batch, total_k, num_heads).bytes;
}

namespace {
int check_quant_sizes(int batch, int64_t total_k, int num_heads) {
  if (batch < 1 || num_heads < 1 || total_k < 0)
    return fail(MLA_ERR_INVALID_ARG, "batch >= 1, num_heads >= 1, total_k >= 0 required (got %d, %d, %lld)", batch,
                num_heads, (long long)total_k);
  if (num_heads > 65535) return fail(MLA_ERR_INVALID_ARG, "num_heads must be <= 65535");
  // one quantiser workgroup per tile index: total_k / 64 + batch of them
  if (total_k / 64 + batch > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARG, "total_k / 64 + batch exceeds the 32-bit grid");
  return MLA_OK;
}
}  // namespace

int mla_prefill_quantize_kv(const void* k_nope, const void* k_rope, const void* v, const int32_t* cu_seqlens_k,
                            int batch, int64_t total_k, int num_heads, void* qkv, size_t qkv_bytes, void* stream) {
  if (!k_nope || !k_rope || !v || !cu_seqlens_k || !qkv) return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  int st = check_quant_sizes(batch, total_k, num_heads);
  if (st != MLA_OK) return st;
  if (!aligned(k_nope, 16) || !aligned(k_rope, 16) || !aligned(v, 16) || !aligned(qkv, 256))
    return fail(MLA_ERR_INVALID_ARG, "k_nope, k_rope, v must be 16-byte and qkv 256-byte aligned");
  if (!aligned(cu_seqlens_k, 4)) return fail(MLA_ERR_INVALID_ARG, "cu_seqlens_k must be 4-byte aligned");
  const size_t need = mla::qkv_layout(batch, total_k, num_heads).bytes;
  if (qkv_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "qkv buffer too small: %zu bytes, need %zu", qkv_bytes, need);
  DevInfo d;
  st = device_info(&d);
  if (st != MLA_OK) return st;
  hipEvent_t ev0, ev1;
  prof_begin(&ev0, &ev1);
  hipError_t e = mla::launch_quant_kv((const uint16_t*)k_nope, (const uint16_t*)k_rope, (const uint16_t*)v,
                                      cu_seqlens_k, batch, total_k, num_heads, (uint8_t*)qkv, (hipStream_t)stream,
                                      ev0, ev1);
  prof_end(MLA_PROFILE_QUANTIZE, ev0, ev1, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "quantiser launch: %s", hipGetErrorString(e));
  return ok();
}

int mla_prefill_quant_fwd(const void* q, const void* qkv, size_t qkv_bytes, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int batch, int max_q_len, int64_t total_k, int num_heads,
                          float softmax_scale, float* out, float* lse, void* stream) {
  if (!q || !qkv || !cu_seqlens_q || !cu_seqlens_k || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  int st = check_quant_sizes(batch, total_k, num_heads);
  if (st != MLA_OK) return st;
  if (max_q_len < 1) return fail(MLA_ERR_INVALID_ARG, "max_q_len must be >= 1 (got %d)", max_q_len);
  const long long nblk = ((long long)max_q_len + mla::prefill_q8_rows_per_block() - 1) / mla::prefill_q8_rows_per_block();
  if (nblk * batch * num_heads > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARG, "batch * query blocks * num_heads exceeds the 32-bit grid index");
  if (!isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(qkv, 256))
    return fail(MLA_ERR_INVALID_ARG, "q and out must be 16-byte and qkv 256-byte aligned");
  if (!aligned(lse, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return fail(MLA_ERR_INVALID_ARG, "lse and the offsets must be 4-byte aligned");
  const size_t need = mla::qkv_layout(batch, total_k, num_heads).bytes;
  if (qkv_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "qkv buffer too small: %zu bytes, need %zu", qkv_bytes, need);
  DevInfo d;
  st = device_info(&d);
  if (st != MLA_OK) return st;
  hipEvent_t ev0, ev1;
  prof_begin(&ev0, &ev1);
  hipError_t e = mla::launch_prefill_q8((const uint16_t*)q, (const uint8_t*)qkv, cu_seqlens_q, cu_seqlens_k, batch,
                                        max_q_len, total_k, num_heads, softmax_scale, out, lse, (hipStream_t)stream,
                                        ev0, ev1);
  prof_end(MLA_PROFILE_ATTENTION, ev0, ev1, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "quantised prefill launch: %s", hipGetErrorString(e));
  return ok();
}

int mla_combine(const float* part_out, const float* part_lse, const int32_t* seq_part_offsets,
                int batch, int rows_per_seq, float* out, float* lse, void* stream) {
  if (!part_out || !part_lse || !seq_part_offsets || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (batch < 1 || rows_per_seq < 1 || rows_per_seq > MLA_MAX_ROWS)
    return fail(MLA_ERR_INVALID_ARG, "batch >= 1 and 1 <= rows_per_seq <= %d required", MLA_MAX_ROWS);
  if ((long long)batch * rows_per_seq > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARG, "batch * rows_per_seq exceeds the 32-bit row index");
  if (!aligned(part_out, 16) || !aligned(out, 16))
    return fail(MLA_ERR_INVALID_ARG, "part_out and out must be 16-byte aligned");
  if (!aligned(part_lse, 4) || !aligned(lse, 4) || !aligned(seq_part_offsets, 4))
    return fail(MLA_ERR_INVALID_ARG, "part_lse, lse, seq_part_offsets must be 4-byte aligned");
  DevInfo d;
  int st = device_info(&d);
  if (st != MLA_OK) return st;
  hipEvent_t ev0, ev1;
  prof_begin(&ev0, &ev1);
  hipError_t e = mla::launch_combine(part_out, part_lse, seq_part_offsets, nullptr, 1, batch, rows_per_seq,
                                     out, lse, 0, (hipStream_t)stream, nullptr, 0, ev0, ev1);
  prof_end(MLA_PROFILE_COMBINE, ev0, ev1, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int mla_append_kv(const void* latent, int batch, int new_tokens, const int32_t* block_table,
                  int max_pages_per_seq, const int32_t* cache_seqlens, void* kv_cache, float* kv_scale,
                  int kv_dtype, int num_pages, void* stream) {
  if (!latent || !block_table || !cache_seqlens || !kv_cache)
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (batch < 1 || new_tokens < 1 || max_pages_per_seq < 1 || num_pages < 1)
    return fail(MLA_ERR_INVALID_ARG, "batch, new_tokens, max_pages_per_seq, num_pages must be >= 1");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "kv_dtype %d not supported", kv_dtype);
  if (kv_dtype == MLA_KV_FP8_E4M3 && !kv_scale)
    return fail(MLA_ERR_INVALID_ARG, "fp8 cache needs kv_scale");
  if (kv_dtype == MLA_KV_BF16 && kv_scale)
    return fail(MLA_ERR_INVALID_ARG, "kv_scale must be NULL for a bf16 cache");
  if (!aligned(latent, 16) || !aligned(kv_cache, 16))
    return fail(MLA_ERR_INVALID_ARG, "latent and kv_cache must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(cache_seqlens, 4) || (kv_scale && !aligned(kv_scale, 4)))
    return fail(MLA_ERR_INVALID_ARG, "block_table, cache_seqlens, kv_scale must be 4-byte aligned");
  DevInfo d;
  int st = device_info(&d);
  if (st != MLA_OK) return st;
  hipError_t e = mla::launch_append((const uint16_t*)latent, batch, new_tokens, block_table, max_pages_per_seq,
                                    cache_seqlens, (uint8_t*)kv_cache, kv_scale,
                                    kv_dtype == MLA_KV_FP8_E4M3 ? 1 : 0, num_pages, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "append kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int mla_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = enable != 0;
  return ok();
}

int mla_debug_page_violations(int reset, uint64_t* count) {
  if (!count) return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  unsigned a = 0, b = 0;
  hipError_t e = mla::page_violations_kernels(&a, reset != 0);
  if (e == hipErrorNotSupported) return fail(MLA_ERR_UNSUPPORTED, "library built without MLA_DEBUG_BOUNDS");
  if (e == hipSuccess) e = mla::page_violations_so(&b, reset != 0);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "page-violation counters: %s", hipGetErrorString(e));
  *count = (uint64_t)a + b;
  return ok();
}

int mla_profile_read_launches(int kernel, float* ms, int capacity, int* count) {
  if (!count || (capacity > 0 && !ms)) return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (kernel < 0 || kernel >= kProfKinds) return fail(MLA_ERR_INVALID_ARG, "unknown kernel kind %d", kernel);
  if (capacity < 0) return fail(MLA_ERR_INVALID_ARG, "capacity must be >= 0");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  int n = 0;
  int st = MLA_OK;
  for (auto& pr : g_prof.recorded[kernel]) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(pr.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, pr.first, pr.second);
    if (e != hipSuccess) {
      st = fail(MLA_ERR_HIP, "profile event: %s", hipGetErrorString(e));
    } else {
      if (n < capacity) ms[n] = t;
      ++n;
    }
    g_prof.pool.push_back(pr.first);
    g_prof.pool.push_back(pr.second);
  }
  g_prof.recorded[kernel].clear();
  *count = n;
  return st == MLA_OK ? ok() : st;
}

int mla_profile_read(double* total_ms, int* launches) {
  if (!total_ms || !launches) return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  std::vector<float> t;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    t.resize(g_prof.recorded[MLA_PROFILE_ATTENTION].size());
  }
  int n = 0;
  const int st = mla_profile_read_launches(MLA_PROFILE_ATTENTION, t.data(), (int)t.size(), &n);
  double sum = 0.0;
  for (int i = 0; i < n && i < (int)t.size(); ++i) sum += t[i];
  *total_ms = sum;
  *launches = n < (int)t.size() ? n : (int)t.size();
  return st;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// No-allocation decode: the split schedule and the partials live in the
// library's static device buffer (mla_scratch.hip) instead of caller buffers.
// ---------------------------------------------------------------------------
extern "C" {

size_t mla_noalloc_scratch_need(int batch, int q_len, int num_heads, int num_units) {
  if (batch < 1 || q_len < 1 || num_heads < 1 || num_units < 1) return 0;
  const size_t md = (mla_metadata_bytes(batch, num_units) + 255) & ~(size_t)255;
  return md + workspace_need(batch, q_len, num_heads, num_units);
}

int mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                           int num_pages, const int32_t* block_table, int max_pages_per_seq,
                           const int32_t* cache_seqlens, int batch, int q_len, int num_heads,
                           float softmax_scale, float* out, float* lse, int num_units, int min_tiles_per_unit,
                           void* stream) {
  if (batch < 1 || q_len < 1 || num_heads < 1)
    return fail(MLA_ERR_INVALID_ARG, "batch, q_len, num_heads must be >= 1 (got %d, %d, %d)", batch, q_len,
                num_heads);
  if (num_units < 0) return fail(MLA_ERR_INVALID_ARG, "num_units must be >= 0 (got %d)", num_units);
  if (min_tiles_per_unit < 0)
    return fail(MLA_ERR_INVALID_ARG, "min_tiles_per_unit must be >= 0 (got %d)", min_tiles_per_unit);
  if ((long long)q_len * num_heads > MLA_MAX_ROWS)
    return fail(MLA_ERR_INVALID_ARG, "q_len * num_heads = %lld exceeds %d", (long long)q_len * num_heads,
                MLA_MAX_ROWS);
  int units = num_units;
  if (units == 0) {
    units = mla_default_num_units(batch, q_len, num_heads);
    if (units < 1) {
      char why[sizeof(g_err)];
      snprintf(why, sizeof(why), "%s", g_err);
      return fail(MLA_ERR_HIP, "no default unit count: %s", why);
    }
  }
  const size_t need = mla_noalloc_scratch_need(batch, q_len, num_heads, units);
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE, "schedule and partials need %zu bytes; the static scratch holds %zu", need,
                (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  void* base = nullptr;
  e = mla::scratch_address(dev, &base);
  if (e != hipSuccess || !base) return fail(MLA_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  const size_t md_bytes = (mla_metadata_bytes(batch, units) + 255) & ~(size_t)255;
  const int rows = q_len * num_heads;
  const MetadataLaunch ml{min_tiles_per_unit == 0 ? mla::kDefaultMinTiles : min_tiles_per_unit,
                          mla::variant_for(rows) == mla::VAR_NARROW16 ? mla::kSeqCostNarrow : mla::kSeqCostWide};
  return decode_impl(q, nullptr, 0, kv_cache, kv_scale, kv_dtype, num_pages, block_table, max_pages_per_seq,
                     cache_seqlens, batch, q_len, num_heads, softmax_scale, out, lse, base, units,
                     (uint8_t*)base + md_bytes, need - md_bytes, stream, false, &ml);
}

}  // extern "C"
