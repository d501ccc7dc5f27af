// Host-side check of the C ABI's validation, sizing and planning code
// (mla_api.hip), built with AddressSanitizer and UndefinedBehaviorSanitizer
// and run on the CPU. No GPU and no HIP runtime: this file supplies a fake
// device (the HIP calls mla_api.hip makes) and fake kernel launchers that
// record what the library would launch, so every host path -- argument
// errors, device queries, default unit counts, workspace carving, the
// measurement hook -- runs under the sanitizers and its launch parameters are
// checked against the buffers the caller passed.
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "mla_decode.h"
#include "mla_internal.h"

// ------------------------------------------------------------------ fake device
static int g_dev = 0;                       // current device index
static const char* g_arch[3] = {"gfx950:sramecc+:xnack-", "gfx942:sramecc+:xnack-", "gfx950"};
static const int g_cus[3] = {256, 304, 80};
static int g_events = 0;

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = g_dev;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* p, int dev) {
  if (dev < 0 || dev > 2) return hipErrorInvalidDevice;
  memset(p, 0, sizeof(*p));
  strncpy(p->gcnArchName, g_arch[dev], sizeof(p->gcnArchName) - 1);
  p->multiProcessorCount = g_cus[dev];
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "fake HIP error"; }
// The fake runtime owns its event objects (as the HIP runtime does): they
// stay reachable from here for the life of the process.
static unsigned char g_event_store[64][16];
hipError_t hipEventCreate(hipEvent_t* e) {
  if (g_events >= 64) return hipErrorOutOfMemory;
  *e = (hipEvent_t)g_event_store[g_events++];
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.5f;
  return hipSuccess;
}
}

// ------------------------------------------------------------------ fake launchers
struct Launch {
  int kind = 0;   // 1 decode, 2 metadata, 3 append, 4 combine, 5 prefill, 6 quantiser, 7 quantised prefill
  mla::DecodeParams p{};
  int variant = 0, grid_units = 0, batch = 0, units = 0, rows = 0, skip_single = 0, min_tiles = 0, cost = 0;
  const void* a = nullptr;
  const void* b = nullptr;
  bool events = false;
};
static std::vector<Launch> g_launches;
// host stand-in for the static device buffer of the no-allocation entry point
alignas(256) static unsigned char g_scratch[1 << 20];
static int g_scratch_lookups = 0;

namespace mla {
int variant_for(int rows) { return rows <= 16 ? VAR_NARROW16 : VAR_WIDE64X; }
int variant_rows(int variant) { return variant == VAR_NARROW16 ? 16 : 64; }
int prefill_rows_per_block() { return 128; }
hipError_t launch_decode(const DecodeParams& p, int variant, int grid_units, hipStream_t, hipEvent_t e0,
                         hipEvent_t e1) {
  Launch l;
  l.kind = 1;
  l.p = p;
  l.variant = variant;
  l.grid_units = grid_units;
  l.events = e0 && e1;
  g_launches.push_back(l);
  return hipSuccess;
}
hipError_t launch_metadata(const int32_t* seqlens, int batch, int units, int min_tiles, int seq_cost, int32_t* md,
                           hipStream_t, hipEvent_t e0, hipEvent_t e1) {
  Launch l;
  l.kind = 2;
  l.events = e0 && e1;
  l.a = seqlens;
  l.b = md;
  l.batch = batch;
  l.units = units;
  l.min_tiles = min_tiles;
  l.cost = seq_cost;
  g_launches.push_back(l);
  return hipSuccess;
}
hipError_t launch_append(const uint16_t*, int batch, int, const int32_t*, int, const int32_t*, uint8_t*, float*,
                         int, int, hipStream_t) {
  Launch l;
  l.kind = 3;
  l.batch = batch;
  g_launches.push_back(l);
  return hipSuccess;
}
hipError_t launch_combine(const float* part_out, const float* part_lse, const int32_t*, const int32_t*, int,
                          int batch, int rows, float*, float*, int skip_single, hipStream_t, const int32_t*,
                          int units, hipEvent_t e0, hipEvent_t e1) {
  Launch l;
  l.kind = 4;
  l.events = e0 && e1;
  l.a = part_out;
  l.b = part_lse;
  l.batch = batch;
  l.rows = rows;
  l.skip_single = skip_single;
  l.units = units;
  g_launches.push_back(l);
  return hipSuccess;
}
hipError_t launch_prefill(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*,
                          const int32_t*, int batch, int, int, float, float*, float*, hipStream_t, hipEvent_t e0,
                          hipEvent_t e1) {
  Launch l;
  l.kind = 5;
  l.batch = batch;
  l.events = e0 && e1;
  g_launches.push_back(l);
  return hipSuccess;
}
int prefill_q8_rows_per_block() { return 128; }
hipError_t launch_quant_kv(const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, int batch,
                           long long total_k, int, uint8_t* qkv, hipStream_t, hipEvent_t e0, hipEvent_t e1) {
  Launch l;
  l.kind = 6;
  l.batch = batch;
  l.units = (int)total_k;
  l.a = qkv;
  l.events = e0 && e1;
  g_launches.push_back(l);
  return hipSuccess;
}
hipError_t launch_prefill_q8(const uint16_t*, const uint8_t* qkv, const int32_t*, const int32_t*, int batch, int,
                             long long total_k, int, float, float*, float*, hipStream_t, hipEvent_t e0,
                             hipEvent_t e1) {
  Launch l;
  l.kind = 7;
  l.batch = batch;
  l.units = (int)total_k;
  l.a = qkv;
  l.events = e0 && e1;
  g_launches.push_back(l);
  return hipSuccess;
}
hipError_t page_violations_kernels(unsigned* c, bool) { *c = 0; return hipErrorNotSupported; }
hipError_t page_violations_so(unsigned* c, bool) { *c = 0; return hipErrorNotSupported; }
hipError_t scratch_address(int dev, void** out) {
  ++g_scratch_lookups;
  *out = dev == g_dev ? g_scratch : nullptr;
  return dev == g_dev ? hipSuccess : hipErrorInvalidDevice;
}
}  // namespace mla

// ------------------------------------------------------------------ checks
static int g_fail = 0;
#define CHECK(cond)                                                                \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      fprintf(stderr, "%s:%d: CHECK failed: %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
              mla_last_error());                                                   \
      ++g_fail;                                                                    \
    }                                                                              \
  } while (0)

// Host buffers standing in for device memory (never dereferenced by the
// library on the host; sized so that the recorded pointers can be checked
// against them).
alignas(256) static unsigned char g_buf[8][1 << 16];

struct DecodeCall {
  const void* q = g_buf[0];
  const void* kv = g_buf[1];
  const float* scale = nullptr;
  int dtype = MLA_KV_BF16, pages = 8;
  const int32_t* bt = (const int32_t*)g_buf[2];
  int maxp = 4;
  const int32_t* sl = (const int32_t*)g_buf[3];
  int B = 2, s = 1, H = 16;
  float sm = 0.072f;
  float* out = (float*)g_buf[4];
  float* lse = (float*)g_buf[5];
  const void* md = nullptr;
  int units = 0;
  void* ws = nullptr;
  size_t wsb = 0;
  int run() const {
    return mla_decode_fwd(q, kv, scale, dtype, pages, bt, maxp, sl, B, s, H, sm, out, lse, md, units, ws, wsb,
                          nullptr);
  }
};

static void check_decode_errors() {
  const unsigned char* odd = g_buf[6] + 4;
  struct Case {
    const char* what;
    void (*mut)(DecodeCall&);
    int expect;
  };
  const Case cases[] = {
      {"q NULL", [](DecodeCall& c) { c.q = nullptr; }, MLA_ERR_INVALID_ARG},
      {"kv NULL", [](DecodeCall& c) { c.kv = nullptr; }, MLA_ERR_INVALID_ARG},
      {"out NULL", [](DecodeCall& c) { c.out = nullptr; }, MLA_ERR_INVALID_ARG},
      {"lse NULL", [](DecodeCall& c) { c.lse = nullptr; }, MLA_ERR_INVALID_ARG},
      {"batch 0", [](DecodeCall& c) { c.B = 0; }, MLA_ERR_INVALID_ARG},
      {"q_len 0", [](DecodeCall& c) { c.s = 0; }, MLA_ERR_INVALID_ARG},
      {"heads 0", [](DecodeCall& c) { c.H = 0; }, MLA_ERR_INVALID_ARG},
      {"rows 4097", [](DecodeCall& c) { c.H = 4097; }, MLA_ERR_INVALID_ARG},
      {"rows huge", [](DecodeCall& c) { c.s = 1 << 20; c.H = 1 << 20; }, MLA_ERR_INVALID_ARG},
      {"pages 0", [](DecodeCall& c) { c.pages = 0; }, MLA_ERR_INVALID_ARG},
      {"max_pages 0", [](DecodeCall& c) { c.maxp = 0; }, MLA_ERR_INVALID_ARG},
      {"scale nan", [](DecodeCall& c) { c.sm = __builtin_nanf(""); }, MLA_ERR_INVALID_ARG},
      {"scale inf", [](DecodeCall& c) { c.sm = __builtin_inff(); }, MLA_ERR_INVALID_ARG},
      {"dtype 7", [](DecodeCall& c) { c.dtype = 7; }, MLA_ERR_UNSUPPORTED},
      {"fp8 no scale", [](DecodeCall& c) { c.dtype = MLA_KV_FP8_E4M3; }, MLA_ERR_INVALID_ARG},
      {"md, units 0", [](DecodeCall& c) { c.md = g_buf[6]; c.ws = g_buf[7]; c.wsb = 1 << 16; }, MLA_ERR_INVALID_ARG},
      {"md, no ws", [](DecodeCall& c) { c.md = g_buf[6]; c.units = 8; }, MLA_ERR_INVALID_ARG},
      {"md, small ws", [](DecodeCall& c) { c.md = g_buf[6]; c.units = 8; c.ws = g_buf[7]; c.wsb = 1024; },
       MLA_ERR_WORKSPACE},
  };
  for (const Case& k : cases) {
    DecodeCall c;
    k.mut(c);
    const size_t before = g_launches.size();
    const int st = c.run();
    if (st != k.expect) fprintf(stderr, "decode case '%s': status %d, expected %d\n", k.what, st, k.expect);
    CHECK(st == k.expect);
    CHECK(strlen(mla_last_error()) > 0);
    CHECK(g_launches.size() == before);   // nothing launched on an argument error
  }
  // misaligned pointers
  DecodeCall c;
  c.q = odd;
  CHECK(c.run() == MLA_ERR_INVALID_ARG);
  c = DecodeCall();
  c.out = (float*)(g_buf[4] + 4);
  CHECK(c.run() == MLA_ERR_INVALID_ARG);
  c = DecodeCall();
  c.lse = (float*)(g_buf[5] + 2);
  CHECK(c.run() == MLA_ERR_INVALID_ARG);
}

// A valid split call carves the caller's workspace into partial O and LSE
// without leaving it, and launches the attention kernel then the merge.
static void check_decode_plan(int B, int s, int H, int units, int dtype) {
  static std::vector<unsigned char> ws;
  const size_t need = mla_workspace_bytes(B, s, H, units);
  CHECK(need > 0);
  ws.assign(need + 256, 0);
  unsigned char* base = (unsigned char*)(((uintptr_t)ws.data() + 255) & ~(uintptr_t)255);
  DecodeCall c;
  c.B = B;
  c.s = s;
  c.H = H;
  c.dtype = dtype;
  c.scale = dtype == MLA_KV_FP8_E4M3 ? (const float*)g_buf[6] : nullptr;
  c.md = g_buf[6];
  c.units = units;
  c.ws = base;
  c.wsb = need;
  g_launches.clear();
  CHECK(c.run() == MLA_OK);
  CHECK(strlen(mla_last_error()) == 0);
  CHECK(g_launches.size() == 2);
  if (g_launches.size() != 2) return;
  const Launch& d = g_launches[0];
  const Launch& m = g_launches[1];
  CHECK(d.kind == 1 && m.kind == 4);
  const size_t rows = (size_t)s * H;
  const size_t slots = (size_t)B + units;
  CHECK(d.p.rows == (int)rows && d.p.batch == B && d.p.q_len == s && d.p.num_heads == H);
  CHECK(d.grid_units == units);
  CHECK(d.variant == (rows <= 16 ? mla::VAR_NARROW16 : mla::VAR_WIDE64X));
  CHECK((dtype == MLA_KV_FP8_E4M3) == (d.p.kv_scale != nullptr));
  const unsigned char* o0 = (const unsigned char*)d.p.ws_out;
  const unsigned char* l0 = (const unsigned char*)d.p.ws_lse;
  CHECK(o0 == base);
  CHECK(l0 >= o0 + slots * rows * 512 * sizeof(float));
  CHECK(l0 + slots * rows * sizeof(float) <= base + need);
  CHECK(((uintptr_t)l0 % 16) == 0);
  CHECK(m.a == d.p.ws_out && m.b == d.p.ws_lse && m.batch == B && m.rows == (int)rows && m.units == units);
  CHECK(m.skip_single == 1);
  CHECK(d.p.scale_log2 > 0.1038f && d.p.scale_log2 < 0.1039f);   // 0.072 * log2(e)
}

static void check_unsplit_and_variants() {
  DecodeCall c;
  g_launches.clear();
  CHECK(c.run() == MLA_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].kind == 1);
  if (!g_launches.empty()) {
    CHECK(g_launches[0].grid_units == c.B);          // one unit per sequence
    CHECK(g_launches[0].p.ws_out == nullptr && g_launches[0].p.md == nullptr);
  }
  // fp8-MFMA entry point: fp8 cache only, 64-row variant at any row count
  g_launches.clear();
  CHECK(mla_decode_fwd_fp8mma(c.q, c.kv, (const float*)g_buf[6], MLA_KV_FP8_E4M3, 8, c.bt, 4, c.sl, 2, 1, 16,
                              0.072f, c.out, c.lse, nullptr, 0, nullptr, 0, nullptr) == MLA_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].variant == mla::VAR_Q8);
  CHECK(mla_decode_fwd_fp8mma(c.q, c.kv, nullptr, MLA_KV_BF16, 8, c.bt, 4, c.sl, 2, 1, 16, 0.072f, c.out, c.lse,
                              nullptr, 0, nullptr, 0, nullptr) == MLA_ERR_UNSUPPORTED);
  // varlen: rows of q are total_q * H, the largest count sizes the row blocks
  g_launches.clear();
  CHECK(mla_decode_fwd_varlen(c.q, (const int32_t*)g_buf[6], 7, 3, c.kv, nullptr, MLA_KV_BF16, 8, c.bt, 4, c.sl, 2,
                              64, 0.072f, c.out, c.lse, nullptr, 0, nullptr, 0, nullptr) == MLA_OK);
  CHECK(g_launches.size() == 1);
  if (!g_launches.empty()) {
    CHECK(g_launches[0].p.q_rows == 7 * 64 && g_launches[0].p.rows == 3 * 64);
    CHECK(g_launches[0].p.cu_q == (const int32_t*)g_buf[6]);
  }
  CHECK(mla_decode_fwd_varlen(c.q, nullptr, 7, 3, c.kv, nullptr, 0, 8, c.bt, 4, c.sl, 2, 64, 0.072f, c.out, c.lse,
                              nullptr, 0, nullptr, 0, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd_varlen(c.q, (const int32_t*)g_buf[6], 0, 3, c.kv, nullptr, 0, 8, c.bt, 4, c.sl, 2, 64,
                              0.072f, c.out, c.lse, nullptr, 0, nullptr, 0, nullptr) == MLA_ERR_INVALID_ARG);
}

static void check_sizes_and_defaults() {
  CHECK(mla_abi_version() == MLA_ABI_VERSION);
  CHECK(strcmp(mla_status_string(MLA_OK), "MLA_OK") == 0);
  CHECK(strcmp(mla_status_string(12345), "MLA_ERR_UNKNOWN") == 0);
  CHECK(mla_metadata_bytes(0, 8) == 0 && mla_metadata_bytes(8, 0) == 0);
  CHECK(mla_metadata_bytes(64, 256) == (size_t)(8 + 3 * 64 + 2 + 2 * 256 + 1) * 4);
  CHECK(mla_workspace_bytes(0, 1, 16, 8) == 0);
  // (batch + units) * rows * 512 * 4 + the LSE block rounded up to 256 bytes
  CHECK(mla_workspace_bytes(64, 1, 16, 256) == (size_t)320 * 16 * 2048 + ((320 * 16 * 4 + 255) / 256) * 256);
  // large shapes do not overflow 32-bit arithmetic
  CHECK(mla_workspace_bytes(1 << 20, 32, 128, 1 << 16) > ((size_t)1 << 40));
  // default unit counts on a 256-CU device (8 XCDs of 32 CUs): k units per
  // XCD fill whole rounds of k * rb workgroups
  g_dev = 0;
  CHECK(mla_default_num_units(64, 1, 16) == 256);     // rb 1: 32 units per XCD
  CHECK(mla_default_num_units(128, 2, 128) == 64);    // rb 4: 8 per XCD, 32 workgroups
  CHECK(mla_default_num_units(128, 6, 128) == 64);    // rb 12: k = 8, 96 workgroups = 3 rounds
  CHECK(mla_default_num_units(128, 3, 64) == 256);    // rb 3: k = 32, 96 workgroups
  // varlen: k also >= ceil(batch / 8), rounded up to a step of 32 / gcd(32, rb)
  CHECK(mla_default_num_units_varlen(128, 6, 128) == 128);   // rb 12: k >= 16, step 8
  CHECK(mla_default_num_units_varlen(1000, 1, 128) == 1024); // rb 2: k >= 125, step 16
  CHECK(mla_default_num_units(0, 1, 16) == 0);
  // another device: 80 CUs = 10 per XCD
  g_dev = 2;
  CHECK(mla_default_num_units(64, 1, 16) == 80);
  CHECK(mla_default_num_units(128, 2, 128) == 40);    // rb 4: k = 5 (10 / gcd(10, 4) = 5)
  g_dev = 0;
}

static void check_unsupported_device() {
  g_dev = 1;   // gfx942
  DecodeCall c;
  g_launches.clear();
  CHECK(c.run() == MLA_ERR_UNSUPPORTED);
  CHECK(strstr(mla_last_error(), "gfx942") != nullptr);
  CHECK(mla_default_num_units(64, 1, 16) == 0);
  CHECK(g_launches.empty());
  g_dev = 0;
}

static void check_metadata_and_others() {
  const int32_t* sl = (const int32_t*)g_buf[3];
  int32_t* md = (int32_t*)g_buf[6];
  const size_t mdb = mla_metadata_bytes(64, 256);
  CHECK(mla_get_split_metadata(nullptr, 64, 1, 16, 256, 0, md, mdb, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_get_split_metadata(sl, 64, 1, 16, 256, -1, md, mdb, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_get_split_metadata(sl, 64, 1, 16, 256, 0, md, mdb - 4, nullptr) == MLA_ERR_WORKSPACE);
  CHECK(mla_get_split_metadata(sl, 64, 1, 16, 256, 0, (int32_t*)(g_buf[6] + 2), mdb, nullptr) ==
        MLA_ERR_INVALID_ARG);
  g_launches.clear();
  CHECK(mla_get_split_metadata(sl, 64, 1, 16, 256, 0, md, mdb, nullptr) == MLA_OK);
  CHECK(mla_get_split_metadata(sl, 64, 2, 128, 256, 5, md, mdb, nullptr) == MLA_OK);
  CHECK(g_launches.size() == 2);
  if (g_launches.size() == 2) {
    CHECK(g_launches[0].min_tiles == mla::kDefaultMinTiles && g_launches[0].cost == mla::kSeqCostNarrow);
    CHECK(g_launches[1].min_tiles == 5 && g_launches[1].cost == mla::kSeqCostWide);
  }
  // combine
  g_launches.clear();
  const float* po = (const float*)g_buf[0];
  CHECK(mla_combine(po, po, sl, 2, 16, (float*)g_buf[4], (float*)g_buf[5], nullptr) == MLA_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].skip_single == 0);
  CHECK(mla_combine(po, po, sl, 2, 4097, (float*)g_buf[4], (float*)g_buf[5], nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_combine(nullptr, po, sl, 2, 16, (float*)g_buf[4], (float*)g_buf[5], nullptr) == MLA_ERR_INVALID_ARG);
  // append
  CHECK(mla_append_kv(g_buf[0], 2, 1, sl, 4, sl, g_buf[1], nullptr, MLA_KV_BF16, 8, nullptr) == MLA_OK);
  CHECK(mla_append_kv(g_buf[0], 2, 1, sl, 4, sl, g_buf[1], (float*)g_buf[6], MLA_KV_BF16, 8, nullptr) ==
        MLA_ERR_INVALID_ARG);
  CHECK(mla_append_kv(g_buf[0], 2, 1, sl, 4, sl, g_buf[1], nullptr, MLA_KV_FP8_E4M3, 8, nullptr) ==
        MLA_ERR_INVALID_ARG);
  // prefill, including the 32-bit workgroup index bound
  const uint16_t* q = (const uint16_t*)g_buf[0];
  CHECK(mla_prefill_fwd(q, q, q, q, sl, sl, 2, 1024, 16, 0.072f, (float*)g_buf[4], (float*)g_buf[5], nullptr) ==
        MLA_OK);
  CHECK(mla_prefill_fwd(q, q, q, q, sl, sl, 40000, 1 << 15, 256, 0.072f, (float*)g_buf[4], (float*)g_buf[5],
                        nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_prefill_fwd(q, q, q, q, sl, sl, 2, 1024, 70000, 0.072f, (float*)g_buf[4], (float*)g_buf[5],
                        nullptr) == MLA_ERR_INVALID_ARG);

  // quantised prefill: buffer size, layout bound, errors
  // 100 keys, 2 sequences -> 100/64 + 2 = 3 slots per head
  const size_t need = mla_prefill_quant_kv_bytes(2, 100, 2);
  CHECK(need == 3 * 2 * 12288 + 3 * 2 * 8192 + 3 * 2 * 256 + 256);
  CHECK(mla_prefill_quant_kv_bytes(0, 100, 2) == 0 && mla_prefill_quant_kv_bytes(2, -1, 2) == 0);
  void* qkv = g_buf[6];
  g_launches.clear();
  CHECK(mla_prefill_quantize_kv(q, q, q, sl, 2, 100, 2, qkv, need - 1, nullptr) == MLA_ERR_WORKSPACE);
  CHECK(mla_prefill_quantize_kv(q, q, q, sl, 1, 10, 1, qkv, mla_prefill_quant_kv_bytes(1, 10, 1), nullptr) == MLA_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].kind == 6 && g_launches[0].units == 10 && g_launches[0].a == qkv);
  CHECK(mla_prefill_quantize_kv(q, q, q, sl, 1, 10, 1, qkv, mla_prefill_quant_kv_bytes(1, 10, 1) - 1, nullptr) ==
        MLA_ERR_WORKSPACE);
  CHECK(mla_prefill_quantize_kv(q, q, q, sl, 1, 10, 1, (char*)qkv + 16, 1 << 15, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_prefill_quantize_kv(q, q, q, sl, 1, 10, 70000, qkv, 1 << 15, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_prefill_quantize_kv(q, q, q, sl, 1, (int64_t)1 << 40, 1, qkv, 1 << 15, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_prefill_quantize_kv(nullptr, q, q, sl, 1, 10, 1, qkv, 1 << 15, nullptr) == MLA_ERR_INVALID_ARG);
  const size_t n1 = mla_prefill_quant_kv_bytes(1, 10, 1);
  CHECK(mla_prefill_quant_fwd(q, qkv, n1, sl, sl, 1, 10, 10, 1, 0.072f, (float*)g_buf[4], (float*)g_buf[5],
                              nullptr) == MLA_OK);
  CHECK(g_launches.back().kind == 7 && g_launches.back().units == 10);
  CHECK(mla_prefill_quant_fwd(q, qkv, n1 - 1, sl, sl, 1, 10, 10, 1, 0.072f, (float*)g_buf[4], (float*)g_buf[5],
                              nullptr) == MLA_ERR_WORKSPACE);
  CHECK(mla_prefill_quant_fwd(q, qkv, n1, sl, sl, 1, 0, 10, 1, 0.072f, (float*)g_buf[4], (float*)g_buf[5],
                              nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_prefill_quant_fwd(q, qkv, 1 << 30, sl, sl, 40000, 1 << 15, 10, 256, 0.072f, (float*)g_buf[4],
                              (float*)g_buf[5], nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_prefill_quant_fwd(q, qkv, n1, sl, sl, 1, 10, 10, 1, INFINITY, (float*)g_buf[4], (float*)g_buf[5],
                              nullptr) == MLA_ERR_INVALID_ARG);

  // page-id bounds counters: a library built without the page-id checks has none
  uint64_t nviol = 7;
  CHECK(mla_debug_page_violations(1, &nviol) == MLA_ERR_UNSUPPORTED);
  CHECK(mla_debug_page_violations(1, nullptr) == MLA_ERR_INVALID_ARG);
}

static void check_profile_hook() {
  double ms = -1.0;
  int n = -1;
  CHECK(mla_profile_read(nullptr, &n) == MLA_ERR_INVALID_ARG);
  CHECK(mla_profile_enable(1) == MLA_OK);
  DecodeCall c;
  g_launches.clear();
  for (int i = 0; i < 3; ++i) CHECK(c.run() == MLA_OK);
  CHECK(g_launches.size() == 3 && g_launches[0].events);
  CHECK(mla_profile_enable(0) == MLA_OK);
  CHECK(c.run() == MLA_OK);   // not recorded
  CHECK(mla_profile_read(&ms, &n) == MLA_OK);
  CHECK(n == 3 && ms > 1.49 && ms < 1.51);
  CHECK(mla_profile_read(&ms, &n) == MLA_OK && n == 0 && ms == 0.0);
  const int created = g_events;
  CHECK(mla_profile_enable(1) == MLA_OK);
  CHECK(c.run() == MLA_OK);
  CHECK(mla_profile_enable(0) == MLA_OK);
  CHECK(g_events == created);   // events come back to the pool and are reused
  CHECK(mla_profile_read(&ms, &n) == MLA_OK && n == 1);
  // per-kind records: a split call records the attention kernel and the
  // merge, the planner its kernel; each kind is read and cleared on its own
  static std::vector<unsigned char> ws(mla_workspace_bytes(2, 1, 16, 4) + 256);
  c.md = g_buf[6];
  c.units = 4;
  c.ws = (void*)(((uintptr_t)ws.data() + 255) & ~(uintptr_t)255);
  c.wsb = mla_workspace_bytes(2, 1, 16, 4);
  CHECK(mla_profile_enable(1) == MLA_OK);
  g_launches.clear();
  CHECK(c.run() == MLA_OK && c.run() == MLA_OK);
  CHECK(mla_get_split_metadata(c.sl, 2, 1, 16, 4, 0, g_buf[6], mla_metadata_bytes(2, 4), nullptr) == MLA_OK);
  CHECK(mla_profile_enable(0) == MLA_OK);
  CHECK(g_launches.size() == 5);
  for (const Launch& l : g_launches) CHECK(l.events);
  float t[4] = {0, 0, 0, 0};
  CHECK(mla_profile_read_launches(MLA_PROFILE_COMBINE, t, 1, &n) == MLA_OK && n == 2 && t[0] == 0.5f && t[1] == 0);
  CHECK(mla_profile_read_launches(MLA_PROFILE_METADATA, t, 4, &n) == MLA_OK && n == 1);
  CHECK(mla_profile_read_launches(MLA_PROFILE_ATTENTION, nullptr, 0, &n) == MLA_OK && n == 2);
  CHECK(mla_profile_read_launches(MLA_PROFILE_ATTENTION, t, 4, &n) == MLA_OK && n == 0);
  CHECK(mla_profile_read_launches(4, t, 4, &n) == MLA_ERR_INVALID_ARG);
  CHECK(mla_profile_read_launches(0, nullptr, 4, &n) == MLA_ERR_INVALID_ARG);
  // the pool grows only to the most pairs held at once (5 launches here)
  CHECK(g_events <= 10);
}

// The no-allocation entry point: size limit checked before any launch; the
// schedule and the partials are carved from the scratch without overlap.
static void check_noalloc() {
  DecodeCall c;
  CHECK(mla_noalloc_scratch_need(0, 1, 16, 8) == 0);
  const size_t need = mla_noalloc_scratch_need(2, 1, 16, 8);
  CHECK(need == ((mla_metadata_bytes(2, 8) + 255) & ~(size_t)255) + mla_workspace_bytes(2, 1, 16, 8));
  // the fp8 workload at the default unit count fits; a much larger shape does not
  CHECK(mla_noalloc_scratch_need(128, 2, 128, 64) <= (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  g_launches.clear();
  CHECK(mla_decode_fwd_noalloc(c.q, c.kv, nullptr, 0, 8, c.bt, 4, c.sl, 1024, 8, 128, 0.072f, c.out, c.lse, 0, 0,
                               nullptr) == MLA_ERR_WORKSPACE);
  CHECK(mla_decode_fwd_noalloc(c.q, c.kv, nullptr, 0, 8, c.bt, 4, c.sl, 2, 1, 16, 0.072f, c.out, c.lse, -1, 0,
                               nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd_noalloc(c.q, c.kv, nullptr, 0, 8, c.bt, 4, c.sl, 2, 1, 16, 0.072f, c.out, c.lse, 8, -1,
                               nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd_noalloc(nullptr, c.kv, nullptr, 0, 8, c.bt, 4, c.sl, 2, 1, 16, 0.072f, c.out, c.lse, 8, 0,
                               nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(g_launches.empty());   // nothing launched on an error
  CHECK(mla_decode_fwd_noalloc(c.q, c.kv, nullptr, 0, 8, c.bt, 4, c.sl, 2, 1, 16, 0.072f, c.out, c.lse, 8, 0,
                               nullptr) == MLA_OK);
  CHECK(g_launches.size() == 3);
  if (g_launches.size() == 3) {
    const Launch& m = g_launches[0];
    const Launch& d = g_launches[1];
    const Launch& cb = g_launches[2];
    CHECK(m.kind == 2 && d.kind == 1 && cb.kind == 4);
    CHECK(m.b == (const void*)g_scratch && d.p.md == (const int32_t*)g_scratch);
    CHECK(m.units == 8 && d.grid_units == 8 && m.min_tiles == mla::kDefaultMinTiles);
    const unsigned char* o0 = (const unsigned char*)d.p.ws_out;
    CHECK(o0 >= g_scratch + mla_metadata_bytes(2, 8) && ((uintptr_t)o0 % 256) == 0);
    CHECK((const unsigned char*)d.p.ws_lse + (size_t)10 * 16 * 4 <= g_scratch + need);
  }
  // default unit count on the 256-CU device
  g_launches.clear();
  CHECK(mla_decode_fwd_noalloc(c.q, c.kv, nullptr, 0, 8, c.bt, 4, c.sl, 64, 1, 16, 0.072f, c.out, c.lse, 0, 3,
                               nullptr) == MLA_OK);
  CHECK(g_launches.size() == 3 && g_launches[1].grid_units == 256 && g_launches[0].min_tiles == 3);
  CHECK(g_scratch_lookups >= 2);
}

int main() {
  check_sizes_and_defaults();
  check_decode_errors();
  check_unsplit_and_variants();
  for (int dtype : {MLA_KV_BF16, MLA_KV_FP8_E4M3}) {
    check_decode_plan(2, 1, 16, 8, dtype);
    check_decode_plan(64, 1, 16, 256, dtype);
    check_decode_plan(128, 2, 128, 64, dtype);
    check_decode_plan(3, 32, 128, 5, dtype);
    check_decode_plan(1000, 5, 64, 1024, dtype);
  }
  check_unsupported_device();
  check_metadata_and_others();
  check_profile_hook();
  check_noalloc();
  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("abi host check: all checks passed\n");
  return 0;
}
